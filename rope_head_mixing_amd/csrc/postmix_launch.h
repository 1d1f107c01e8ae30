// postmix_launch.h -- internal interface between the C ABI layer and the
// gfx950 kernels.  Not installed; the public interface is include/postmix.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pm {

struct MixArgs {
    const uint16_t* X;      // O (forward) or dY (input gradient)
    const uint16_t* W;
    const float* rcos;
    const float* rsin;
    int64_t table_rows;
    const int32_t* positions;
    int64_t sq;
    int nh, nope, pe;
    uint16_t* Out;          // Y or dO
    int n_cu;               // compute units of the device
    int waves_per_cu;       // resident single-wave workgroups to aim for per CU
    bool force_general;     // use the general (persistent) kernel for every shape
};

struct DwArgs {
    const uint16_t* dY;
    const uint16_t* O;
    const float* rcos;
    const float* rsin;
    int64_t table_rows;
    const int32_t* positions;
    int64_t sq;
    int nh, nope, pe;
    float* dW;
    float* partials;        // [partials, nh, nh] fp32 workspace (dw_plan or bwd_fused_plan)
    bool force_general;     // use the direct-load kernel for every shape
};

hipError_t launch_mix(const MixArgs& a, bool dx, hipStream_t stream);
int mix_part_width(int64_t sq, int nh, int nope, int pe);
hipError_t launch_dw(const DwArgs& a, hipStream_t stream);
hipError_t launch_kv_remap(const int32_t* idx, int64_t rows, int64_t sq, int64_t topk,
                           int64_t seqlen_kv, int32_t pad, int32_t* out, hipStream_t stream);
hipError_t launch_rope_apply(const uint16_t* X, const float* rcos, const float* rsin, int64_t table_rows,
                             const int32_t* positions, int64_t sq, int nh, int nope, int pe, int direction,
                             uint16_t* Out, hipStream_t stream);
hipError_t launch_rope_table(double theta, int pe, int64_t rows, float* cos_out, float* sin_out,
                             int n_cu, hipStream_t stream);

// Partition of the weight gradient into partials: token blocks, each split
// into `spans` channel spans (1 unless the accumulation chain of a block would
// be too long).  A function of the shape only, so the summation order (and
// therefore every bit of dW) does not depend on the GPU.
struct DwPlan {
    int64_t blocks;
    int spans;
    int64_t partials() const { return blocks * spans; }
};
int dw_tokens_per_block(int64_t sq, int nh);
int64_t dw_num_blocks(int64_t sq, int nh);
DwPlan dw_plan(int64_t sq, int nh, int nope, int pe);         // postmix_bwd_dw
DwPlan bwd_fused_plan(int64_t sq, int nh, int nope, int pe);  // postmix_bwd's single pass
int bwd_fused_tokens_per_block(int64_t sq, int nh, int nope, int pe);
int dw_chunk_width(int nh, int nope, int pe);

// Fused backward: dx (into mx.Out) and the dW partials from one pass over dY
// and O, then the reduce into a.dW.  Only for shapes where bwd_fused_applies.
bool bwd_fused_applies(int nh, int nope, int pe);
hipError_t launch_bwd_fused(const MixArgs& mx, const DwArgs& a, hipStream_t stream);

}  // namespace pm
