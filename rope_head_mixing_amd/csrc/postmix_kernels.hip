// postmix_kernels.hip -- gfx950 (MI355X) kernels for the fused inverse-RoPE +
// VHA postmix (PaddleFleet PR #1772, "Fuse HCA inverse RoPE into the VHA
// postmix, and the sparse-attention KV index remap", PR body item 1).
//
// Shapes: activations [sq, nh, d] bf16 with d = nope + pe, channel fastest;
// W [nh, nh] bf16 with W[g,h], g the output head; RoPE tables fp32
// [rows, pe/2]; positions int32 [sq].
//
// MFMA used throughout: v_mfma_f32_32x32x16_bf16 (wave64).
//   A operand: lane l supplies row (l % 32) and 8 k-values.
//   B operand: lane l supplies column (l % 32) and 8 k-values.
//   D (16 fp32 per lane): register r of lane l is row 8*(r/4) + 4*(l/32) + r%4,
//   column l % 32.
// The products are summed over k, so which 8 k-values sit in which lane half
// only has to agree between A and B; the kernels assign k freely.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "postmix_launch.h"

namespace pm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// scalar helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16, round to nearest even.  gfx950 converts in hardware
// (v_cvt_pk_bf16_f32); for every finite float its result equals the bit-level
// definition u += 0x7fff + ((u >> 16) & 1), u >> 16 (checked exhaustively on
// the device over all 2^32 bit patterns).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// two floats rounded to bf16 and packed, a in the low half (one instruction)
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    const bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t pack2(uint32_t lo16, uint32_t hi16) {
    return (lo16 & 0xffffu) | (hi16 << 16);
}

// Weight-gradient pe operand of 2*NW channels (NW packed bf16 pairs):
// x_k = a_k C_k + b_k S_k (own value a, rotation partner b, S already
// signed), split into the bf16 pair hi = RNE(x), lo = RNE(x - hi) of the
// compensated product.
template <int NW>
__device__ __forceinline__ void rotate_split(const uint32_t* own, const uint32_t* par, const float* cs,
                                             const float* sn, uint32_t* hi, uint32_t* lo) {
#pragma unroll
    for (int jj = 0; jj < NW; ++jj) {
        float x[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int k = 2 * jj + e;
            const float xa = __uint_as_float(e ? (own[jj] & 0xffff0000u) : (own[jj] << 16));
            const float xb = __uint_as_float(e ? (par[jj] & 0xffff0000u) : (par[jj] << 16));
            x[e] = xa * cs[k] + xb * sn[k];
        }
        const uint32_t h = pack_bf16(x[0], x[1]);
        hi[jj] = h;
        lo[jj] = pack_bf16(x[0] - __uint_as_float(h << 16), x[1] - __uint_as_float(h & 0xffff0000u));
    }
}

__device__ __forceinline__ void rotate_split8(const uint32_t* own, const uint32_t* par, const float* cs,
                                              const float* sn, uint32_t* hi, uint32_t* lo) {
    rotate_split<4>(own, par, cs, sn, hi, lo);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ int64_t table_row(const int32_t* positions, int64_t s,
                                             int64_t table_rows) {
    int64_t p = positions[s];
    p = p < 0 ? 0 : p;
    return p >= table_rows ? table_rows - 1 : p;
}

// Data-sized launches.  One dimension of a dispatch holds fewer than 2^32
// work-items, so a grid of more than 2^21 workgroups (2^31 work-items at 1024
// threads) takes rows of 2^21 in x and the rows in y: workgroup
// b = y * 2^21 + x.  The fixed row width keeps gridDim out of the index (on
// gfx950 reading it costs a dispatch-packet load and a division).  The last
// row can run past n: each such kernel checks its index.
constexpr int kGridXLog2 = 21;
constexpr int64_t kMaxGridY = 65535;
static bool data_grid(int64_t n_blocks, dim3* g) {
    const int64_t gx = (int64_t)1 << kGridXLog2;
    if (n_blocks <= gx) {
        *g = dim3((unsigned)n_blocks);
        return true;
    }
    const int64_t gy = (n_blocks + gx - 1) / gx;
    if (gy > kMaxGridY) return false;
    *g = dim3((unsigned)gx, (unsigned)gy);
    return true;
}

// workgroup index; ROWS = false for a grid of one row, where it is blockIdx.x
template <bool ROWS = true>
__device__ __forceinline__ int64_t linear_block() {
    if constexpr (ROWS) return ((int64_t)blockIdx.y << kGridXLog2) + blockIdx.x;
    return blockIdx.x;
}

// ---------------------------------------------------------------------------
// channel groups
//
// Channels are handled in groups of 8 (one 16-byte vector).  A "unit" is two
// groups that one MFMA lane half owns together (slot 0 and slot 1):
//   nope units u < NU:   slot s covers channels 16u + 8s .. +8 (valid if < nope)
//   pe units u = NU + t: slot 0 covers nope + 8t .. +8 (first rotation half),
//                        slot 1 covers nope + pe/2 + 8t .. +8 (its partners).
// So a rotation partner always sits in the same lane, register r <-> r + 8.
// ---------------------------------------------------------------------------

struct ChanMap {
    int nope, h2, nu_nope, n_units;
    __device__ __forceinline__ ChanMap(int nope_, int pe_) {
        nope = nope_;
        h2 = pe_ >> 1;
        nu_nope = (nope_ + 15) >> 4;
        n_units = nu_nope + (h2 >> 3);
    }
    // first channel of (unit, slot), or -1 for padding
    __device__ __forceinline__ int base(int u, int slot) const {
        if (u < nu_nope) {
            int c = 16 * u + 8 * slot;
            return c < nope ? c : -1;
        }
        if (u < n_units) return nope + 8 * (u - nu_nope) + slot * h2;
        return -1;
    }
    __device__ __forceinline__ bool is_pe(int u) const { return u >= nu_nope && u < n_units; }
};

// ---------------------------------------------------------------------------
// head-mix kernel (forward and input gradient)
//
//   forward:  Y[s,g,:]  = inv_rope( sum_h W[g,h] X[s,h,:] ),   X = O
//   dx:       dO[s,h,:] = rope    ( sum_g W[g,h] X[s,g,:] ),   X = dY
//
// One wave per workgroup; the workgroup strides over work items.  A work item
// is one token s and MPI M-blocks (each M-block = 2 units = 32 channels).  Its
// [NHP x 32*MPI] tile of X is loaded with coalesced 16-byte loads (prefetched
// one item ahead in registers), staged in LDS, and read back transposed into
// MFMA A fragments (rows = channels, k = heads).  W^T (or W for dx) is the B
// operand, held in registers for the whole kernel.  The fp32 accumulators of
// the pe units are rotated in registers, rounded to bf16 and stored as
// 16-byte vectors.
// ---------------------------------------------------------------------------

template <int NHP, int MPI, bool DX>
__global__ __launch_bounds__(64) void mix_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
    const float* __restrict__ rcos, const float* __restrict__ rsin, int64_t table_rows,
    const int32_t* __restrict__ positions, int nh, int nope, int pe,
    uint16_t* __restrict__ Out, int64_t total_items, int items_per_token) {
    constexpr int KB = NHP / 16;            // k-blocks of 16 heads
    constexpr int NB = (NHP + 31) / 32;     // output blocks of 32 heads
    constexpr int GPI = 4 * MPI;            // channel groups per item
    constexpr int PITCH = GPI * 8 + 8;      // LDS row pitch (bf16), 16 B pad
    constexpr int LOADS = NHP * GPI / 64;   // 16-byte loads per lane per item
    static_assert(NHP % 16 == 0 && (NHP * GPI) % 64 == 0, "tile shape");
    __shared__ __attribute__((aligned(16))) uint16_t lds[NHP * PITCH];

    const int lane = threadIdx.x;
    const int d = nope + pe;
    const ChanMap cm(nope, pe);

    // B operand (k = contracted head, n = output head), all of W in registers.
    bf16x8 wf[KB][NB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int n = 32 * nb + (lane & 31);
            u32x4 v;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                uint32_t two[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int k = 16 * kb + 8 * (lane >> 5) + 2 * jj + e;
                    const int g = DX ? k : n;  // row of W (output head of the forward)
                    const int h = DX ? n : k;  // column of W
                    two[e] = (g < nh && h < nh) ? (uint32_t)W[g * nh + h] : 0u;
                }
                v[jj] = pack2(two[0], two[1]);
            }
            wf[kb][nb] = as_bf16x8(v);
        }

    // A-fragment geometry: lane supplies logical row m = lane % 32, which the
    // D layout places in lane half Q, register r; map it to (group, element).
    const int m = lane & 31;
    const int aQ = (m & 7) >> 2;
    const int ar = 4 * (m >> 3) + (m & 3);
    const int a_col = (aQ * 2 + (ar >> 3)) * 8 + (ar & 7);  // within an M-block
    const int a_h0 = 8 * (lane >> 5);

    u32x4 buf[LOADS];

    auto load_item = [&](int64_t item) {
        const int64_t s = item / items_per_token;
        const int mb0 = (int)(item - s * items_per_token) * MPI;
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int idx = j * 64 + lane;
            const int h = idx / GPI;
            const int grp = idx % GPI;
            const int u = 2 * (mb0 + grp / 4) + ((grp >> 1) & 1);
            const int c = cm.base(u, grp & 1);
            u32x4 v = {0u, 0u, 0u, 0u};
            if (h < nh && c >= 0)
                v = *reinterpret_cast<const u32x4*>(X + ((s * nh + h) * (int64_t)d + c));
            buf[j] = v;
        }
    };

    int64_t item = blockIdx.x;
    if (item < total_items) load_item(item);

    for (; item < total_items; item += gridDim.x) {
        const int64_t s = item / items_per_token;
        const int mb0 = (int)(item - s * items_per_token) * MPI;

        __syncthreads();  // the previous item's LDS reads are complete
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int idx = j * 64 + lane;
            *reinterpret_cast<u32x4*>(&lds[(idx / GPI) * PITCH + (idx % GPI) * 8]) = buf[j];
        }
        __syncthreads();

        const int64_t next = item + gridDim.x;
        if (next < total_items) load_item(next);  // in flight during the compute

        int64_t prow = 0;
        if (pe > 0) prow = table_row(positions, s, table_rows);

#pragma unroll
        for (int mbl = 0; mbl < MPI; ++mbl) {
            f32x16 acc[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[nb][r] = 0.0f;

#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int h0 = 16 * kb + a_h0;
                const uint16_t* p = &lds[h0 * PITCH + mbl * 32 + a_col];
                u32x4 v;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    v[jj] = pack2(p[(2 * jj) * PITCH], p[(2 * jj + 1) * PITCH]);
                const bf16x8 af = as_bf16x8(v);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, wf[kb][nb], acc[nb], 0, 0, 0);
            }

            // epilogue: lane half Q owns unit u; registers 0..7 = slot 0, 8..15 = slot 1
            const int Q = lane >> 5;
            const int u = 2 * (mb0 + mbl) + Q;
            const int c0 = cm.base(u, 0), c1 = cm.base(u, 1);
            float cs[8], sn[8];
            const bool rot = cm.is_pe(u);
            if (rot) {
                const int i0 = 8 * (u - cm.nu_nope);
                const f32x4* pc = reinterpret_cast<const f32x4*>(rcos + prow * cm.h2 + i0);
                const f32x4* ps = reinterpret_cast<const f32x4*>(rsin + prow * cm.h2 + i0);
                const f32x4 ca = pc[0], cb = pc[1], sa = ps[0], sb = ps[1];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    cs[e] = ca[e]; cs[4 + e] = cb[e];
                    sn[e] = sa[e]; sn[4 + e] = sb[e];
                }
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int row = 32 * nb + (lane & 31);  // output head
                float y[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) y[r] = acc[nb][r];
                if (rot) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float z0 = y[e], z1 = y[8 + e];
                        if (DX) {   // RoPE: turn by +phi
                            y[e] = z0 * cs[e] - z1 * sn[e];
                            y[8 + e] = z1 * cs[e] + z0 * sn[e];
                        } else {    // inverse RoPE: turn by -phi
                            y[e] = z0 * cs[e] + z1 * sn[e];
                            y[8 + e] = z1 * cs[e] - z0 * sn[e];
                        }
                    }
                }
                if (row < nh) {
                    uint16_t* orow = Out + (s * nh + row) * (int64_t)d;
                    if (c0 >= 0) {
                        u32x4 v;
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj)
                            v[jj] = pack_bf16(y[2 * jj], y[2 * jj + 1]);
                        *reinterpret_cast<u32x4*>(orow + c0) = v;
                    }
                    if (c1 >= 0) {
                        u32x4 v;
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj)
                            v[jj] = pack_bf16(y[8 + 2 * jj], y[9 + 2 * jj]);
                        *reinterpret_cast<u32x4*>(orow + c1) = v;
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// weight-gradient partial kernel
//
//   P_b[g,h] = sum over tokens s of block b, channels c:
//                  dY[s,g,c] * inv_rope(O)[s,h,c]
//
// MFMA with A = dY rows (m = g), B = inv_rope(O) rows (n = h), k = channels:
// both operands are channel-contiguous, so each lane loads its 8 channels with
// one 16-byte load straight from HBM.  K-step t covers channel groups 2t (lane
// half 0) and 2t+1 (lane half 1).  For a pe group the lane also loads the
// rotation partner group and the cos/sin of its 8 pairs, rotates in fp32 and
// splits the result into bf16 hi + bf16 lo; both are accumulated, which keeps
// the rotated operand to ~2^-17 relative (nope products are exact).
//
// 256 threads (4 waves).  nh <= 64 (NB <= 2): every wave owns all NB x NB
// output tiles and the waves split the block's tokens round-robin; the four
// wave sums are added in the fixed order (w0 + w2) + (w1 + w3) in LDS.
// nh <= 128 (NB = 4): wave w owns the 2 x 2 tiles (g-blocks 2(w/2)+{0,1},
// h-blocks 2(w%2)+{0,1}) over all tokens of the block; no cross-wave sum.
// ---------------------------------------------------------------------------

template <int NHP>
__global__ __launch_bounds__(256) void dw_partial_kernel(
    const uint16_t* __restrict__ dY, const uint16_t* __restrict__ O,
    const float* __restrict__ rcos, const float* __restrict__ rsin, int64_t table_rows,
    const int32_t* __restrict__ positions, int64_t sq, int nh, int nope, int pe,
    float* __restrict__ partials, int spans) {
    constexpr int NB = (NHP + 31) / 32;
    constexpr bool SPLIT_TOKENS = NB <= 2;
    constexpr int TG = SPLIT_TOKENS ? NB : 2;
    constexpr int TH = SPLIT_TOKENS ? NB : 2;
    __shared__ __attribute__((aligned(16))) float red[SPLIT_TOKENS ? 2 * TG * TH * 16 * 64 : 1];

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int gb0 = SPLIT_TOKENS ? 0 : 2 * (wave >> 1);
    const int hb0 = SPLIT_TOKENS ? 0 : 2 * (wave & 1);
    const int d = nope + pe, h2 = pe >> 1;
    const int ngroups = d >> 3;
    const int ksteps = (ngroups + 1) >> 1;
    const int pe_first_step = (nope >> 3) >> 1;  // first k-step holding a pe group
    const int half = lane >> 5;

    f32x16 acc[TG][TH];
#pragma unroll
    for (int a = 0; a < TG; ++a)
#pragma unroll
        for (int b = 0; b < TH; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    // token block tb of B = gridDim.x / spans: tokens [tb*sq/B, (tb+1)*sq/B);
    // k-step span y: [y*ksteps/spans, (y+1)*ksteps/spans) (spans > 1 only
    // for very wide rows, to bound the accumulation chain)
    const int64_t nbt = gridDim.x / spans, tb = blockIdx.x / spans;
    const int y = (int)(blockIdx.x - tb * spans);
    const int64_t s_begin = tb * sq / nbt;
    const int64_t s_end = (tb + 1) * sq / nbt;
    const int t_begin = (int)((int64_t)y * ksteps / spans), t_end = (int)((int64_t)(y + 1) * ksteps / spans);

    for (int64_t s = s_begin + (SPLIT_TOKENS ? wave : 0); s < s_end; s += (SPLIT_TOKENS ? 4 : 1)) {
        int64_t prow = 0;
        if (pe > 0) prow = table_row(positions, s, table_rows);
        const uint16_t* dys = dY + s * nh * (int64_t)d;
        const uint16_t* os = O + s * nh * (int64_t)d;

        for (int t = t_begin; t < t_end; ++t) {
            const int grp = 2 * t + half;
            const int c = 8 * grp;
            const bool gvalid = grp < ngroups;

            bf16x8 a[TG];
#pragma unroll
            for (int tg = 0; tg < TG; ++tg) {
                const int g = 32 * (gb0 + tg) + (lane & 31);
                u32x4 v = {0u, 0u, 0u, 0u};
                if (gvalid && g < nh) v = *reinterpret_cast<const u32x4*>(dys + g * d + c);
                a[tg] = as_bf16x8(v);
            }

            if (t < pe_first_step) {
                // nope channels only: the B operand is O itself (exact bf16)
#pragma unroll
                for (int th = 0; th < TH; ++th) {
                    const int h = 32 * (hb0 + th) + (lane & 31);
                    u32x4 v = {0u, 0u, 0u, 0u};
                    if (gvalid && h < nh) v = *reinterpret_cast<const u32x4*>(os + h * d + c);
                    const bf16x8 b = as_bf16x8(v);
#pragma unroll
                    for (int tg = 0; tg < TG; ++tg)
                        acc[tg][th] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[tg], b, acc[tg][th], 0, 0, 0);
                }
            } else {
                // this k-step may hold pe groups: rotate, split hi/lo
                const bool pe_grp = gvalid && c >= nope;
                const bool first = c < nope + h2;
                const int i0 = first ? c - nope : c - nope - h2;
                const int cpart = first ? c + h2 : c - h2;
                const float sgn = first ? 1.0f : -1.0f;
                float cs[8], sn[8];
                if (pe_grp) {
                    const f32x4* pc = reinterpret_cast<const f32x4*>(rcos + prow * h2 + i0);
                    const f32x4* ps = reinterpret_cast<const f32x4*>(rsin + prow * h2 + i0);
                    const f32x4 ca = pc[0], cb = pc[1], sa = ps[0], sb = ps[1];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        cs[e] = ca[e]; cs[4 + e] = cb[e];
                        sn[e] = sgn * sa[e]; sn[4 + e] = sgn * sb[e];
                    }
                }
#pragma unroll
                for (int th = 0; th < TH; ++th) {
                    const int h = 32 * (hb0 + th) + (lane & 31);
                    u32x4 own = {0u, 0u, 0u, 0u}, part = {0u, 0u, 0u, 0u};
                    if (gvalid && h < nh) {
                        own = *reinterpret_cast<const u32x4*>(os + h * d + c);
                        if (pe_grp) part = *reinterpret_cast<const u32x4*>(os + h * d + cpart);
                    }
                    u32x4 hi = own, lo = {0u, 0u, 0u, 0u};
                    if (pe_grp) {  // first half: a C + b S; second half: a C - b S
                        uint32_t ow[4], pw[4], hw[4], lw[4];
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) { ow[jj] = own[jj]; pw[jj] = part[jj]; }
                        rotate_split8(ow, pw, cs, sn, hw, lw);
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) { hi[jj] = hw[jj]; lo[jj] = lw[jj]; }
                    }
                    const bf16x8 bh = as_bf16x8(hi), bl = as_bf16x8(lo);
#pragma unroll
                    for (int tg = 0; tg < TG; ++tg) {
                        acc[tg][th] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[tg], bh, acc[tg][th], 0, 0, 0);
                        acc[tg][th] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[tg], bl, acc[tg][th], 0, 0, 0);
                    }
                }
            }
        }
    }

    float* part = partials + (int64_t)blockIdx.x * nh * nh;
    if constexpr (SPLIT_TOKENS) {
        // fixed-order sum of the four waves: (w0 + w2) + (w1 + w3)
        auto slot = [&](int w2, int tg, int th, int r) -> float& {
            return red[(((w2 * TG + tg) * TH + th) * 16 + r) * 64 + lane];
        };
        __syncthreads();
        if (wave >= 2) {
#pragma unroll
            for (int tg = 0; tg < TG; ++tg)
#pragma unroll
                for (int th = 0; th < TH; ++th)
#pragma unroll
                    for (int r = 0; r < 16; ++r) slot(wave - 2, tg, th, r) = acc[tg][th][r];
        }
        __syncthreads();
        if (wave < 2) {
#pragma unroll
            for (int tg = 0; tg < TG; ++tg)
#pragma unroll
                for (int th = 0; th < TH; ++th)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[tg][th][r] += slot(wave, tg, th, r);
        }
        __syncthreads();
        if (wave == 1) {
#pragma unroll
            for (int tg = 0; tg < TG; ++tg)
#pragma unroll
                for (int th = 0; th < TH; ++th)
#pragma unroll
                    for (int r = 0; r < 16; ++r) slot(0, tg, th, r) = acc[tg][th][r];
        }
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int tg = 0; tg < TG; ++tg)
#pragma unroll
            for (int th = 0; th < TH; ++th)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[tg][th][r] += slot(0, tg, th, r);
    }
#pragma unroll
    for (int tg = 0; tg < TG; ++tg)
#pragma unroll
        for (int th = 0; th < TH; ++th) {
            const int h = 32 * (hb0 + th) + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int g = 32 * (gb0 + tg) + 8 * (r >> 2) + 4 * half + (r & 3);
                if (g < nh && h < nh) part[g * nh + h] = acc[tg][th][r];
            }
        }
}

// ---------------------------------------------------------------------------
// fixed-order reduction of the partials: dW[e] = sum_b P[b][e]
//
// Workgroup = 64 elements x 16 waves.  Wave w sums the blocks
// [w*n/16, (w+1)*n/16) in batches of 16 (each batch added as a balanced
// binary tree, batches added in order); the 16 wave sums are then added as a
// balanced binary tree in LDS.  The order depends only on n.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(1024) void dw_reduce_kernel(const float* __restrict__ partials,
                                                         int64_t n_blocks, int64_t n_elems,
                                                         float* __restrict__ dW) {
    __shared__ float red[16][64];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t e = (int64_t)blockIdx.x * 64 + lane;
    const int64_t b0 = n_blocks * wave / 16, b1 = n_blocks * (wave + 1) / 16;
    float total = 0.0f;
    if (e < n_elems) {
        for (int64_t b = b0; b < b1; b += 16) {
            float v[16];
#pragma unroll
            for (int k = 0; k < 16; ++k)
                v[k] = (b + k < b1) ? partials[(b + k) * n_elems + e] : 0.0f;
#pragma unroll
            for (int w = 1; w < 16; w *= 2)
#pragma unroll
                for (int k = 0; k < 16; k += 2 * w) v[k] += v[k + w];
            total += v[0];
        }
    }
    red[wave][lane] = total;
    __syncthreads();
    if (wave == 0) {
        float v[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = red[k][lane];
#pragma unroll
        for (int w = 1; w < 16; w *= 2)
#pragma unroll
            for (int k = 0; k < 16; k += 2 * w) v[k] += v[k + w];
        if (e < n_elems) dW[e] = v[0];
    }
}

// ---------------------------------------------------------------------------
// RoPE tables: cos/sin(r * theta^(-2i/pe)) with the angle in fp64
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void rope_table_kernel(double theta, int pe, int64_t rows,
                                                         float* __restrict__ cos_out,
                                                         float* __restrict__ sin_out) {
    const int h2 = pe >> 1;
    const int64_t n = rows * h2;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = idx / h2;
        const int i = (int)(idx - r * h2);
        const double inv_freq = pow(theta, -2.0 * (double)i / (double)pe);
        const double phi = (double)r * inv_freq;
        double sv, cv;
        sincos(phi, &sv, &cv);
        cos_out[idx] = (float)cv;
        sin_out[idx] = (float)sv;
    }
}

// ---------------------------------------------------------------------------
// head-mix kernel, token-part tiles (forward and input gradient), nh in {32, 64, 128}
//
// A tile is (token s, channel part of CP channels): [nh x CP], contiguous per
// row, read with 16-byte non-temporal loads like a copy and written back the
// same way.  One workgroup per tile: the tile's loads are issued into
// registers first, so they are in flight while W is staged.
//   setup: W -> LDS (in the tile's place, rows padded) -> each wave copies its
//          B operand (W^T for the forward, W for dx; the N-blocks of its
//          N-group when the heads are split, NS > 1) into registers.
//   tile:  registers -> LDS tile; each wave owns M-blocks of 32 channels; the
//          A operand (rows = channels, k = heads) comes from the gfx950
//          transposing LDS load ds_read_b64_tr_b16 (in each group of 16
//          lanes, lane i receives T[k0+e][c0+i], e = 0..3, when source lane j
//          points at T[k0 + j/4][c0 + 4*(j%4)]).  Results are rounded and
//          written over the M-block's own tile columns; pe blocks are rotated
//          in registers first (paired pe blocks, below), or, for other pe
//          layouts, go to an fp32 scratch and are rotated in the store phase,
//          which writes whole rows.
// ---------------------------------------------------------------------------

// pe channels that the MFMA epilogue rotates in registers (paired pe blocks, below)
__host__ __device__ __forceinline__ bool pe_pairs_in_blocks(int nope, int pe) {
    return pe > 0 && pe % 32 == 0 && nope % 32 == 0;
}

template <int NH, int CP, int WAVES, int NS = 1, bool PADDED = false>
struct PartCfg {
    static constexpr int KB = NH / 16, NB = NH / 32, NT = 64 * WAVES;
    // NS > 1: wave w computes N-blocks (w % NS)*NBW .. +NBW of M-blocks w/NS, +MSTEP, ...
    static constexpr int NBW = NB / NS, MSTEP = WAVES / NS;
    // bf16 elements per LDS tile row.  128 rows and unpadded 96-row tiles pad
    // 48 B (rows 12 of 64 banks apart: the transposing A-fragment reads 2-way
    // instead of 4-way): in the benchmark's regime the forward at sq = 8192
    // went 385 -> 373 us at nh = 128 and 312 -> 293 us at nh = 96.  Other
    // tiles keep 16 B: no gain at 64 rows, and padded 96-row tiles (nh = 72)
    // measured 10% slower with the wider rows at the same occupancy.
    static constexpr int PITCH = (NH == 128 || (NH == 96 && !PADDED)) ? CP + 24 : CP + 8;
    static constexpr int WPITCH = NH + 8;                // bf16 elements per LDS row of W
    static constexpr int VPR = CP / 8;                   // 16-byte vectors per tile row
    static constexpr int VPT = NH * VPR / NT;            // vectors per thread
    static constexpr int WVPR = NH / 8;                  // 16-byte vectors per row of W
    static constexpr int WVPT = (NH * WVPR + NT - 1) / NT;
    static constexpr int MBP = CP / 32;                  // M-blocks per part
    static_assert(NH % 32 == 0 && CP % 32 == 0 && (NH * VPR) % NT == 0 && CP >= NH, "part tile shape");
    static_assert(NB % NS == 0 && WAVES % NS == 0 && MBP % MSTEP == 0, "N split");
    // fp32 pe scratch: only for pe layouts that are not rotated in registers
    __host__ __device__ static size_t aux_bytes(int nope, int pe) {
        return pe_pairs_in_blocks(nope, pe) ? 0 : (size_t)NH * (pe + 4) * 4;
    }
    // tile (W is staged there first), then the pe scratch, then the cos and
    // sin rows (pe/2 floats each) of the tile's tp tokens
    __host__ __device__ static size_t lds_bytes(int nope, int pe, int tp = 1) {
        return (size_t)NH * PITCH * 2 + aux_bytes(nope, pe) + (size_t)tp * pe * 4;
    }
    // tokens per tile for nh < NH heads: as many as fill the rows, while each
    // cos/sin quad of every token has a thread to load it
    __host__ __device__ static int tokens_per_tile(int nh, int pe) {
        int tp = NH / nh;
        if (pe > 0 && tp * (pe / 4) > NT) tp = NT / (pe / 4);
        return tp < 1 ? 1 : tp;
    }
};

typedef short i16x4 __attribute__((ext_vector_type(4)));

// lane's 8 k-values of an MFMA operand from a row-major [k][n] LDS matrix:
// rows k0 .. k0+7 are split 4 + 4 over two transposing loads; the lane group
// g = lane/16 takes columns 16*(g%2) .. +16 of the 32-column block and
// k rows 8*(g/2) .. +8 of the 16-row k-block.
// tr_frag2: the same with the two 16-column halves taken from column bases
// clo (lanes of groups 0, 2) and chi (groups 1, 3) of row-major `base`, so
// MFMA rows 0..15 are columns clo.. and rows 16..31 columns chi..
__device__ __forceinline__ bf16x8 tr_frag2(const uint16_t* base, int clo, int chi, int pitch, int lane) {
    const int g = lane >> 4, i = lane & 15;
    const uint16_t* p = base + (8 * (g >> 1) + (i >> 2)) * pitch + ((g & 1) ? chi : clo) + 4 * (i & 3);
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * pitch));
    u32x4 v;
    v[0] = pack2((uint16_t)lo[0], (uint16_t)lo[1]);
    v[1] = pack2((uint16_t)lo[2], (uint16_t)lo[3]);
    v[2] = pack2((uint16_t)hi[0], (uint16_t)hi[1]);
    v[3] = pack2((uint16_t)hi[2], (uint16_t)hi[3]);
    return as_bf16x8(v);
}

__device__ __forceinline__ bf16x8 tr_frag(const uint16_t* base, int pitch, int lane) {
    return tr_frag2(base, 0, 16, pitch, lane);
}

// Paired pe blocks.  When pe % 32 == 0 and nope % 32 == 0 the pe channels of
// a tile form pe/32 MFMA M-blocks whose 32 rows are 16 first-half channels
// (nope + 16q ..) and their 16 rotation partners (nope + pe/2 + 16q ..).  In
// the 32x32 accumulator layout a lane then holds each partner pair in
// registers r and r + 8 (rows 8(r/4) + 4Q + r%4 and that + 16), so the
// rotation happens in registers and the results are rounded to bf16 at once:
// no fp32 scratch, and the store phase is one plain copy for every vector.

// Rotate a paired block's accumulators and write both halves (bf16) into
// row-major `out` (pitch in elements) at local pe offset L (first pe channel):
// first half  i: y = x_i C + sg (x_{i+h2} S),  second half: y = x_{i+h2} C - sg (x_i S),
// sg = +1 for the inverse rotation (-phi), -1 for the rotation by +phi.
__device__ __forceinline__ void rotate_paired_block(const f32x16& acc, uint16_t* out, int pitch, int row,
                                                    int L, int h2, int q, int Q, const float* csl,
                                                    const float* snl, float sg) {
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const int i = 16 * q + 8 * a + 4 * Q;  // 4 consecutive indices within a half
        const f32x4 c4 = *reinterpret_cast<const f32x4*>(csl + i);
        const f32x4 s4 = *reinterpret_cast<const f32x4*>(snl + i);
        float y1[4], y2[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float x1 = acc[4 * a + e], x2 = acc[4 * a + 8 + e];
            y1[e] = x1 * c4[e] + sg * (x2 * s4[e]);
            y2[e] = x2 * c4[e] + (-sg) * (x1 * s4[e]);
        }
        uint2 o1, o2;
        o1.x = pack_bf16(y1[0], y1[1]);
        o1.y = pack_bf16(y1[2], y1[3]);
        o2.x = pack_bf16(y2[0], y2[1]);
        o2.y = pack_bf16(y2[2], y2[3]);
        *reinterpret_cast<uint2*>(out + row * pitch + L + i) = o1;
        *reinterpret_cast<uint2*>(out + row * pitch + L + h2 + i) = o2;
    }
}

template <int NH, int CP, int WAVES, bool DX, int NS, bool PAD>
__global__ __launch_bounds__(64 * WAVES) void mix_part_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
    const float* __restrict__ rcos, const float* __restrict__ rsin, int64_t table_rows,
    const int32_t* __restrict__ positions, int64_t sq, int nh, int nope, int pe, int cpt, int ptok,
    int64_t n_tiles, uint16_t* __restrict__ Out) {
    // PAD: nh < NH.  A tile then holds ptok consecutive tokens (their ptok*nh
    // head rows are consecutive rows of the [sq*nh, d] array) and W is staged
    // block-diagonally, one copy per token; rows beyond the tokens' rows are
    // zero padding, never loaded from or stored to HBM.  Otherwise nh == NH
    // and ptok == 1.
    const int tp = PAD ? ptok : 1;
    using C = PartCfg<NH, CP, WAVES, NS, PAD>;
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    uint16_t* tile = smem;                                   // [NH][PITCH] bf16
    uint16_t* wl = smem;                                     // [NH][WPITCH] bf16 first, in the tile's place
    float* pes = reinterpret_cast<float*>(smem + NH * C::PITCH);  // [NH][pe + 4] fp32 (unpaired pe)
    const int pes_pitch = pe + 4;
    // cos and sin rows of the tile's tokens: [tp][pe] floats (cos then sin)
    float* csl = reinterpret_cast<float*>(reinterpret_cast<char*>(pes) + C::aux_bytes(nope, pe));
    float* snl = csl + (pe >> 1);

    const int d = nope + pe;
    const int h2 = pe >> 1;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar registers

    int64_t t = linear_block();
    u32x4 v[C::VPT];
    // thread tid < tp*pe/4 carries quad tid%(pe/4) of token tid/(pe/4)'s cos
    // (first pe/8 quads) or sin row
    f32x4 rope_v = {0.f, 0.f, 0.f, 0.f};
    int rows_valid = NH;  // head rows of this tile backed by tokens < sq
    auto load_tile = [&](int64_t tt) {
        const int64_t grp = tt / cpt;
        const int part = (int)(tt - grp * cpt);
        const int64_t s0 = grp * tp;
        const int64_t ntok = sq - s0 < tp ? sq - s0 : tp;
        rows_valid = PAD ? (int)ntok * nh : NH;
        const uint16_t* xs = X + s0 * nh * (int64_t)d + part * CP;
        const int q4n = pe >> 2;
        if (pe > 0 && (part + 1) * CP > nope && tid < (int)ntok * q4n) {
            const int p = tid / q4n, q = tid - p * q4n;
            const int64_t prow = table_row(positions, s0 + p, table_rows);
            const int half4 = pe >> 3;
            rope_v = reinterpret_cast<const f32x4*>((q < half4 ? rcos : rsin) + prow * h2)[q < half4 ? q : q - half4];
        }
#pragma unroll
        for (int j = 0; j < C::VPT; ++j) {
            const int q = j * C::NT + tid;
            const int row = q / C::VPR, c8 = q % C::VPR;
            if (!PAD || row < rows_valid)
                v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xs + row * (int64_t)d + 8 * c8));
            else
                v[j] = u32x4{0u, 0u, 0u, 0u};
        }
    };
    // W's loads go out before the tile's: loads complete in issue order, so
    // W issued behind the tile made the W setup (LDS writes, two barriers,
    // fragment reads) wait for the whole tile instead of overlapping it
    u32x4 wv[PAD ? 1 : C::WVPT];
    if (!PAD) {
#pragma unroll
        for (int j = 0; j < C::WVPT; ++j) {
            const int q = j * C::NT + tid;
            if (q < NH * C::WVPR) wv[j] = reinterpret_cast<const u32x4*>(W)[q];
        }
    }
    if (t < n_tiles) load_tile(t);  // the tile's loads overlap the W setup

    // setup: W -> LDS -> B operand in registers
    if (!PAD) {  // 16-byte rows
#pragma unroll
        for (int j = 0; j < C::WVPT; ++j) {
            const int q = j * C::NT + tid;
            if (q < NH * C::WVPR) {
                const int row = q / C::WVPR, c8 = q % C::WVPR;
                *reinterpret_cast<u32x4*>(wl + row * C::WPITCH + 8 * c8) = wv[j];
            }
        }
    } else {  // zero the padded rows, then scatter W's nh*nh elements (16-byte loads when aligned)
        for (int q = tid; q < NH * C::WPITCH / 8; q += C::NT) reinterpret_cast<u32x4*>(wl)[q] = u32x4{0u, 0u, 0u, 0u};
        __syncthreads();
        const int n = nh * nh;
        const int nvec = ((uintptr_t)W & 15u) == 0 ? n / 8 : 0;
        const int bd = nh * (C::WPITCH + 1);  // one block-diagonal step: nh rows and nh columns
        // a work item is one vector of W for one diagonal copy p (tp copies),
        // then one leftover element for one copy: with few heads the copies,
        // not the elements, give the threads their work
        for (int it = tid; it < tp * nvec; it += C::NT) {
            const int p = it / nvec, q = it - p * nvec;
            const u32x4 x = reinterpret_cast<const u32x4*>(W)[q];
            int row = (8 * q) / nh, col = 8 * q - row * nh;
            uint16_t* const blk = wl + p * bd;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                blk[row * C::WPITCH + col] = (uint16_t)(x[e >> 1] >> (16 * (e & 1)));
                if (++col == nh) { col = 0; ++row; }
            }
        }
        const int rem = n - 8 * nvec;
        for (int it = tid; it < tp * rem; it += C::NT) {
            const int p = it / rem, idx = 8 * nvec + (it - p * rem);
            const int row = idx / nh;
            wl[p * bd + row * C::WPITCH + (idx - row * nh)] = W[idx];
        }
    }
    __syncthreads();
    const int ng = wave % NS;  // this wave's N-group: N-blocks ng*NBW .. +NBW
    bf16x8 wf[C::KB][C::NBW];
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int j = 0; j < C::NBW; ++j) {
            const int nb = ng * C::NBW + j;
            if (DX) {  // B[k=g][n=h] = W[g][h]
                wf[kb][j] = tr_frag(wl + (16 * kb) * C::WPITCH + 32 * nb, C::WPITCH, lane);
            } else {   // B[k=h][n=g] = W[g][h]
                const int g = 32 * nb + (lane & 31), h = 16 * kb + 8 * (lane >> 5);
                wf[kb][j] = *reinterpret_cast<const bf16x8*>(wl + g * C::WPITCH + h);
            }
        }
    __syncthreads();  // W's LDS becomes the tile

    const int Q = lane >> 5;
    if (t < n_tiles) {
        const int64_t grp = t / cpt;
        const int part = (int)(t - grp * cpt);
        const int64_t s0 = grp * tp;  // first token of the tile
        const int c_base = part * CP;

#pragma unroll
        for (int j = 0; j < C::VPT; ++j) {
            const int q = j * C::NT + tid;
            const int row = q / C::VPR, c8 = q % C::VPR;
            *reinterpret_cast<u32x4*>(tile + row * C::PITCH + 8 * c8) = v[j];
        }
        const bool tile_pe = pe > 0 && c_base + CP > nope;
        if (tile_pe && tid < tp * (pe >> 2)) reinterpret_cast<f32x4*>(csl)[tid] = rope_v;  // [tp][cos, sin]
        __syncthreads();
        const bool paired = tile_pe && pe_pairs_in_blocks(nope, pe);
        const int L = nope - c_base;  // local index of the first pe channel (tiles with pe)

        // One M-block at a time (64 rows; padded 96-row tiles, with a barrier
        // per block, see below).  This loop is kept as written rather than
        // through mix_block/write_block of the grouped path: routed through
        // them, the 64-row dx measured 2% slower (351 -> 358 us).
        if constexpr (NS == 1 || (NS == 3 && PAD)) {
            for (int b = wave / NS; b < C::MBP; b += C::MSTEP) {
                f32x16 acc[C::NBW];
#pragma unroll
                for (int j = 0; j < C::NBW; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
                const bool pb = paired && 32 * b >= L;  // a paired pe block (wave-uniform)
                const int q = b - (L >> 5);
                const int clo = pb ? L + 16 * q : 32 * b, chi = pb ? L + h2 + 16 * q : 32 * b + 16;
                bf16x8 af[C::KB];
#pragma unroll
                for (int kb = 0; kb < C::KB; ++kb)
                    af[kb] = tr_frag2(tile + (16 * kb) * C::PITCH, clo, chi, C::PITCH, lane);
#pragma unroll
                for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
                    for (int j = 0; j < C::NBW; ++j)
                        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kb], wf[kb][j], acc[j], 0, 0, 0);
                // with an N split, other waves read this M-block's columns too: all
                // reads are done before any wave overwrites them with results
                if (NS > 1) __syncthreads();
                if (pb) {
#pragma unroll
                    for (int j = 0; j < C::NBW; ++j) {
                        const int g = 32 * (ng * C::NBW + j) + (lane & 31);
                        int p = PAD ? g / nh : 0;  // the row's token within the tile
                        p = p < tp ? p : tp - 1;   // (padding rows: any staged row)
                        rotate_paired_block(acc[j], tile, C::PITCH, g, L, h2, q, Q, csl + p * pe, snl + p * pe,
                                            DX ? -1.0f : 1.0f);
                    }
                    continue;
                }
                // D register r of lane half Q: channel 32b + 8(r/4) + 4Q + r%4, head 32nb + lane%32
#pragma unroll
                for (int j = 0; j < C::NBW; ++j) {
                    const int nb = ng * C::NBW + j;
                    const int g = 32 * nb + (lane & 31);
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        const int cl = 32 * b + 8 * a + 4 * Q;  // 4 consecutive channels, all nope or all pe
                        const int cg = c_base + cl;
                        if (cg < nope) {
                            uint2 o;
                            o.x = pack_bf16(acc[j][4 * a], acc[j][4 * a + 1]);
                            o.y = pack_bf16(acc[j][4 * a + 2], acc[j][4 * a + 3]);
                            *reinterpret_cast<uint2*>(tile + g * C::PITCH + cl) = o;
                        } else {
                            f32x4 o = {acc[j][4 * a], acc[j][4 * a + 1], acc[j][4 * a + 2], acc[j][4 * a + 3]};
                            *reinterpret_cast<f32x4*>(pes + g * pes_pitch + (cg - nope)) = o;
                        }
                    }
                }
            }
        } else {
            // one M-block b: its NBW accumulators (MFMA over the heads), then the
            // rounded results written over the block's own tile columns (paired
            // pe blocks rotated in registers first; other pe channels to the fp32
            // scratch)
            auto mix_block = [&](int b, f32x16* acc) {
#pragma unroll
                for (int j = 0; j < C::NBW; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
                const bool pb = paired && 32 * b >= L;  // a paired pe block (wave-uniform)
                const int q = b - (L >> 5);
                const int clo = pb ? L + 16 * q : 32 * b, chi = pb ? L + h2 + 16 * q : 32 * b + 16;
                bf16x8 af[C::KB];
#pragma unroll
                for (int kb = 0; kb < C::KB; ++kb)
                    af[kb] = tr_frag2(tile + (16 * kb) * C::PITCH, clo, chi, C::PITCH, lane);
#pragma unroll
                for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
                    for (int j = 0; j < C::NBW; ++j)
                        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kb], wf[kb][j], acc[j], 0, 0, 0);
            };
            auto write_block = [&](int b, const f32x16* acc) {
                const bool pb = paired && 32 * b >= L;
                const int q = b - (L >> 5);
                if (pb) {
#pragma unroll
                    for (int j = 0; j < C::NBW; ++j) {
                        const int g = 32 * (ng * C::NBW + j) + (lane & 31);
                        int p = PAD ? g / nh : 0;  // the row's token within the tile
                        p = p < tp ? p : tp - 1;   // (padding rows: any staged row)
                        rotate_paired_block(acc[j], tile, C::PITCH, g, L, h2, q, Q, csl + p * pe, snl + p * pe,
                                            DX ? -1.0f : 1.0f);
                    }
                    return;
                }
                // D register r of lane half Q: channel 32b + 8(r/4) + 4Q + r%4, head 32nb + lane%32
#pragma unroll
                for (int j = 0; j < C::NBW; ++j) {
                    const int nb = ng * C::NBW + j;
                    const int g = 32 * nb + (lane & 31);
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        const int cl = 32 * b + 8 * a + 4 * Q;  // 4 consecutive channels, all nope or all pe
                        const int cg = c_base + cl;
                        if (cg < nope) {
                            uint2 o;
                            o.x = pack_bf16(acc[j][4 * a], acc[j][4 * a + 1]);
                            o.y = pack_bf16(acc[j][4 * a + 2], acc[j][4 * a + 3]);
                            *reinterpret_cast<uint2*>(tile + g * C::PITCH + cl) = o;
                        } else {
                            f32x4 o = {acc[j][4 * a], acc[j][4 * a + 1], acc[j][4 * a + 2], acc[j][4 * a + 3]};
                            *reinterpret_cast<f32x4*>(pes + g * pes_pitch + (cg - nope)) = o;
                        }
                    }
                }
            };
            // With an N split, other waves read this wave's M-blocks too, so a
            // block's results wait for a barrier.  The wave's M-blocks go in
            // groups of MG: a group is computed, then one barrier, then its
            // results are written.  128 rows take all four blocks at once, 96
            // rows two: their accumulators fit the registers that the
            // LDS-bound occupancy leaves (two workgroups per CU at 128 rows,
            // three at 96).  Against a barrier per block: nh = 128 fwd 388 ->
            // 375 us, nh = 112 507 -> 462 us, nh = 96 391 -> 372 us.  Padded
            // 96-row tiles measured slower grouped (nh = 80: 401 -> 504 us
            // with two blocks, 551 us with four) and keep a barrier per block.
            constexpr int NMB = C::MBP / C::MSTEP;
            constexpr int MG = NS == 4 ? NMB : 2;
            static_assert(NMB % MG == 0, "M-block groups");
#pragma unroll
            for (int g0 = 0; g0 < NMB; g0 += MG) {
                f32x16 acc[MG][C::NBW];
#pragma unroll
                for (int i = 0; i < MG; ++i) mix_block(wave / NS + (g0 + i) * C::MSTEP, acc[i]);
                __syncthreads();
#pragma unroll
                for (int i = 0; i < MG; ++i) write_block(wave / NS + (g0 + i) * C::MSTEP, acc[i]);
            }
        }
        __syncthreads();

        // store phase: whole rows of the part; pe pairs rotated here
        uint16_t* outs = Out + s0 * nh * (int64_t)d + c_base;
#pragma unroll
        for (int j = 0; j < C::VPT; ++j) {
            const int q = j * C::NT + tid;
            const int row = q / C::VPR, c8 = q % C::VPR;
            if (PAD && row >= rows_valid) continue;  // padding rows
            const int cl = 8 * c8, cg = c_base + cl;
            u32x4 o;
            if (cg < nope || paired) {
                o = *reinterpret_cast<const u32x4*>(tile + row * C::PITCH + cl);
            } else {
                const int i = cg - nope;
                const bool first = i < h2;
                const int ii = first ? i : i - h2;
                const float* own = pes + row * pes_pitch + i;
                const float* par = pes + row * pes_pitch + (first ? i + h2 : i - h2);
                const int rp = PAD ? (row / nh) * pe : 0;  // the row's token's cos/sin
                const f32x4 o0 = reinterpret_cast<const f32x4*>(own)[0], o1 = reinterpret_cast<const f32x4*>(own)[1];
                const f32x4 p0 = reinterpret_cast<const f32x4*>(par)[0], p1 = reinterpret_cast<const f32x4*>(par)[1];
                const f32x4 c0 = reinterpret_cast<const f32x4*>(csl + rp + ii)[0];
                const f32x4 c1 = reinterpret_cast<const f32x4*>(csl + rp + ii)[1];
                const f32x4 sn0 = reinterpret_cast<const f32x4*>(snl + rp + ii)[0];
                const f32x4 sn1 = reinterpret_cast<const f32x4*>(snl + rp + ii)[1];
                // forward (turn by -phi): first half  a C + b S, second half b C - a S
                // dx      (turn by +phi): first half  a C - b S, second half b C + a S
                const float sg = (first != DX) ? 1.0f : -1.0f;
                float y[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    y[e] = o0[e] * c0[e] + sg * (p0[e] * sn0[e]);
                    y[4 + e] = o1[e] * c1[e] + sg * (p1[e] * sn1[e]);
                }
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) o[jj] = pack_bf16(y[2 * jj], y[2 * jj + 1]);
            }
            __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(outs + row * (int64_t)d + cl));
        }
    }
}

// ---------------------------------------------------------------------------
// weight-gradient partial kernel, LDS-staged chunks (nh in {32, 64, 128})
//
// Same partition as dw_partial_kernel (block b = tokens [b*T, (b+1)*T), one
// fp32 partial per block), but the block's data streams through LDS in chunks
// of (token, CH channels): the dY and O rows of a chunk are read with
// coalesced 16-byte non-temporal loads (prefetched one chunk ahead in
// registers), and the MFMA fragments are read from LDS (channels are the
// contraction axis, so no transpose is needed).  A pe group's rotation
// partner lies in the same chunk (the pe range never crosses a chunk), so it
// costs an LDS read, not an HBM read; the chunk's cos/sin rows are staged in
// LDS too.
// nh <= 64: the four waves split each chunk's k-steps and hold every output
// tile; their sums are added in the fixed order (w0 + w2) + (w1 + w3).
// nh == 128: wave w owns the 2 x 2 tiles (g-blocks 2(w/2)+{0,1}, h-blocks
// 2(w%2)+{0,1}) over every k-step.
// ---------------------------------------------------------------------------

template <int NH, int CH>
struct DwCfg {
    // nh <= 64: 4 waves split the k-steps; nh = 128: 8 waves own 2 output tiles each
    static constexpr int NB = NH / 32;
    static constexpr bool SPLIT_K = NB <= 2;
    static constexpr int WAVES = SPLIT_K ? 4 : 8, NT = 64 * WAVES;
    static constexpr int TG = SPLIT_K ? NB : 2, TH = SPLIT_K ? NB : NB * NB / (WAVES * TG);
    static constexpr int PITCH = CH + 8;
    static constexpr int VPR = CH / 8;
    static constexpr int VPO = NH * VPR;           // vectors per operand per chunk
    static constexpr int VPT = 2 * VPO / NT;       // vectors per thread per chunk
    static constexpr int KS = CH / 16;
    static constexpr int KSW = SPLIT_K ? KS / WAVES : KS;
    static constexpr int MAX_H2 = CH / 2;
    static_assert(VPO % NT == 0 && KS % WAVES == 0, "chunk shape");
};

template <int NH, int CH, bool PAD>
__global__ __launch_bounds__((DwCfg<NH, CH>::NT)) void dw_chunk_kernel(
    const uint16_t* __restrict__ dY, const uint16_t* __restrict__ O,
    const float* __restrict__ rcos, const float* __restrict__ rsin, int64_t table_rows,
    const int32_t* __restrict__ positions, int64_t sq, int nh, int nope, int pe,
    float* __restrict__ partials, int ptok, int spans) {
    // PAD: nh < NH.  A chunk then holds ptok consecutive tokens (ptok*nh
    // consecutive rows of the [sq*nh, d] arrays), the rest of its rows are
    // zero padding (not loaded), and the partial is the sum of the ptok
    // diagonal [nh, nh] blocks of the chunk products; otherwise nh == NH and
    // ptok == 1.
    // spans: workgroup b covers token block b / spans and channel span
    // b % spans (its share of each token's 128-channel parts); one partial
    // per workgroup.  spans > 1 only where a token block's accumulation
    // chain would otherwise be too long (very wide rows).
    using C = DwCfg<NH, CH>;
    const int tp = PAD ? ptok : 1;
    // cos and sin rows of the chunk's tokens: [tp][pe/2] each
    constexpr int CSN = PAD ? 4 * C::NT : C::MAX_H2;
    // one array: dY chunk, then O chunk; reused at the end for the wave sums
    __shared__ __attribute__((aligned(16))) uint16_t lbuf[2 * NH * C::PITCH];
    uint16_t* const dyl = lbuf;
    uint16_t* const ol = lbuf + NH * C::PITCH;
    __shared__ __attribute__((aligned(16))) float csl[CSN];
    __shared__ __attribute__((aligned(16))) float snl[CSN];

    const int d = nope + pe, h2 = pe >> 1;
    const int cpt = d / CH;
    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar registers
    const int gb0 = C::SPLIT_K ? 0 : C::TG * (wave / (C::NB / C::TH));
    const int hb0 = C::SPLIT_K ? 0 : C::TH * (wave % (C::NB / C::TH));

    // token block tb of B = gridDim.x / spans: tokens [tb*sq/B, (tb+1)*sq/B);
    // channel span y: parts [y*cpt/spans, (y+1)*cpt/spans)
    const int64_t nbt = gridDim.x / spans, tb = blockIdx.x / spans;
    const int y = (int)(blockIdx.x - tb * spans);
    const int64_t s_begin = tb * sq / nbt;
    const int64_t s_end = (tb + 1) * sq / nbt;
    const int p0 = (int)((int64_t)y * cpt / spans), cps = (int)((int64_t)(y + 1) * cpt / spans) - p0;
    const int nchunks = (int)((s_end - s_begin + tp - 1) / tp) * cps;

    f32x16 acc[C::TG][C::TH];
#pragma unroll
    for (int a = 0; a < C::TG; ++a)
#pragma unroll
        for (int b = 0; b < C::TH; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    u32x4 v[C::VPT];
    f32x4 cv = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
    auto load_chunk = [&](int k) {
        const int64_t s = s_begin + (int64_t)(k / cps) * tp;  // first token of the chunk
        const int part = p0 + k % cps;
        const int ntok = (int)(s_end - s < tp ? s_end - s : tp);
        const int rows_valid = PAD ? ntok * nh : NH;
        const int64_t rowbase = s * nh * (int64_t)d + part * CH;
        const int q4n = h2 >> 2;
        if (pe > 0 && (part + 1) * CH > nope && tid < ntok * q4n) {  // before the chunk loads
            const int p = tid / q4n, q = tid - p * q4n;
            const int64_t prow = table_row(positions, s + p, table_rows);
            cv = reinterpret_cast<const f32x4*>(rcos + prow * h2)[q];
            sv = reinterpret_cast<const f32x4*>(rsin + prow * h2)[q];
        }
#pragma unroll
        for (int j = 0; j < C::VPT; ++j) {
            const int q = j * C::NT + tid;
            const int op = q / C::VPO;               // 0: dY, 1: O (compile-time per j)
            const int rem = q % C::VPO;
            const int row = rem / C::VPR, c8 = rem % C::VPR;
            const uint16_t* src = (op == 0 ? dY : O) + rowbase + row * (int64_t)d + 8 * c8;
            v[j] = (!PAD || row < rows_valid) ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src))
                                      : u32x4{0u, 0u, 0u, 0u};
        }
    };

    if (nchunks > 0) load_chunk(0);
    for (int k = 0; k < nchunks; ++k) {
        const int part = p0 + k % cps;
        __syncthreads();  // every wave is done with the previous chunk
#pragma unroll
        for (int j = 0; j < C::VPT; ++j) {
            const int q = j * C::NT + tid;
            const int op = q / C::VPO;
            const int rem = q % C::VPO;
            const int row = rem / C::VPR, c8 = rem % C::VPR;
            *reinterpret_cast<u32x4*>((op == 0 ? dyl : ol) + row * C::PITCH + 8 * c8) = v[j];
        }
        const bool chunk_pe = pe > 0 && (part + 1) * CH > nope;
        if (chunk_pe && tid < tp * (h2 >> 2)) {
            reinterpret_cast<f32x4*>(csl)[tid] = cv;
            reinterpret_cast<f32x4*>(snl)[tid] = sv;
        }
        __syncthreads();
        if (k + 1 < nchunks) load_chunk(k + 1);  // in flight during the compute

#pragma unroll
        for (int kk = 0; kk < C::KSW; ++kk) {
            const int t = C::SPLIT_K ? wave + C::WAVES * kk : kk;
            const int c = 16 * t + 8 * half;          // channel within the chunk
            const int cg = part * CH + c;             // channel within the head
            bf16x8 a[C::TG];
#pragma unroll
            for (int tg = 0; tg < C::TG; ++tg)
                a[tg] = *reinterpret_cast<const bf16x8*>(dyl + (32 * (gb0 + tg) + (lane & 31)) * C::PITCH + c);
            const bool step_pe = chunk_pe && part * CH + 16 * t + 16 > nope;  // wave-uniform
            if (!step_pe) {
#pragma unroll
                for (int th = 0; th < C::TH; ++th) {
                    const bf16x8 b = *reinterpret_cast<const bf16x8*>(ol + (32 * (hb0 + th) + (lane & 31)) * C::PITCH + c);
#pragma unroll
                    for (int tg = 0; tg < C::TG; ++tg)
                        acc[tg][th] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[tg], b, acc[tg][th], 0, 0, 0);
                }
            } else {
                const bool pe_grp = cg >= nope;
                const bool first = cg < nope + h2;
                const int i0 = first ? cg - nope : cg - nope - h2;
                const int cpart = first ? c + h2 : c - h2;
                const float sgn = first ? 1.0f : -1.0f;
                float cs[8], sn[8];
                if (pe_grp && !PAD) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        cs[e] = csl[i0 + e];
                        sn[e] = sgn * snl[i0 + e];
                    }
                }
#pragma unroll
                for (int th = 0; th < C::TH; ++th) {
                    const int h = 32 * (hb0 + th) + (lane & 31);
                    const u32x4 own = *reinterpret_cast<const u32x4*>(ol + h * C::PITCH + c);
                    u32x4 hi = own, lo = {0u, 0u, 0u, 0u};
                    if (pe_grp && PAD) {  // the angles of row h's token
                        int p = h / nh;
                        p = p < tp ? p : tp - 1;  // (padding rows: any staged row)
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            cs[e] = csl[p * h2 + i0 + e];
                            sn[e] = sgn * snl[p * h2 + i0 + e];
                        }
                    }
                    if (pe_grp) {
                        const u32x4 par = *reinterpret_cast<const u32x4*>(ol + h * C::PITCH + cpart);
                        uint32_t ow[4], pw[4], hw[4], lw[4];
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) { ow[jj] = own[jj]; pw[jj] = par[jj]; }
                        rotate_split8(ow, pw, cs, sn, hw, lw);
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) { hi[jj] = hw[jj]; lo[jj] = lw[jj]; }
                    }
                    const bf16x8 bh = as_bf16x8(hi), bl = as_bf16x8(lo);
#pragma unroll
                    for (int tg = 0; tg < C::TG; ++tg) {
                        acc[tg][th] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[tg], bh, acc[tg][th], 0, 0, 0);
                        acc[tg][th] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[tg], bl, acc[tg][th], 0, 0, 0);
                    }
                }
            }
        }
    }

    float* part_out = partials + (int64_t)blockIdx.x * nh * nh;
    if constexpr (C::SPLIT_K) {
        // fixed-order sum of the four waves, (w0 + w2) + (w1 + w3), in the
        // chunk buffers (2 x TG x TH x 16 x 64 floats fit in dyl + ol)
        float* red = reinterpret_cast<float*>(lbuf);
        static_assert(2 * C::TG * C::TH * 16 * 64 * 4 <= (int)sizeof(lbuf), "reduction area");
        auto slot = [&](int w2, int tg, int th, int r) -> float& {
            return red[(((w2 * C::TG + tg) * C::TH + th) * 16 + r) * 64 + lane];
        };
        __syncthreads();
        if (wave >= 2) {
#pragma unroll
            for (int tg = 0; tg < C::TG; ++tg)
#pragma unroll
                for (int th = 0; th < C::TH; ++th)
#pragma unroll
                    for (int r = 0; r < 16; ++r) slot(wave - 2, tg, th, r) = acc[tg][th][r];
        }
        __syncthreads();
        if (wave < 2) {
#pragma unroll
            for (int tg = 0; tg < C::TG; ++tg)
#pragma unroll
                for (int th = 0; th < C::TH; ++th)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[tg][th][r] += slot(wave, tg, th, r);
        }
        __syncthreads();
        if (wave == 1) {
#pragma unroll
            for (int tg = 0; tg < C::TG; ++tg)
#pragma unroll
                for (int th = 0; th < C::TH; ++th)
#pragma unroll
                    for (int r = 0; r < 16; ++r) slot(0, tg, th, r) = acc[tg][th][r];
        }
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int tg = 0; tg < C::TG; ++tg)
#pragma unroll
            for (int th = 0; th < C::TH; ++th)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[tg][th][r] += slot(0, tg, th, r);
        if (PAD && tp > 1) {
            // several tokens per chunk: the partial is the sum of the diagonal
            // [nh, nh] blocks, p = 0, 1, .. in order, through an [NH][NH+1] matrix
            // in LDS (only this wave is left; its LDS accesses complete in order)
            float* m = reinterpret_cast<float*>(lbuf);
            static_assert(NH * (NH + 1) * 4 <= (int)sizeof(lbuf), "diagonal-block area");
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int tg = 0; tg < C::TG; ++tg)
#pragma unroll
                for (int th = 0; th < C::TH; ++th)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        m[(32 * tg + 8 * (r >> 2) + 4 * half + (r & 3)) * (NH + 1) + 32 * th + (lane & 31)] =
                            acc[tg][th][r];
            __builtin_amdgcn_wave_barrier();
            for (int idx = lane; idx < nh * nh; idx += 64) {
                const int g = idx / nh, h = idx - g * nh;
                float sum = m[g * (NH + 1) + h];
                for (int p = 1; p < tp; ++p) sum += m[(p * nh + g) * (NH + 1) + p * nh + h];
                part_out[idx] = sum;
            }
            return;
        }
    }
#pragma unroll
    for (int tg = 0; tg < C::TG; ++tg)
#pragma unroll
        for (int th = 0; th < C::TH; ++th) {
            const int h = 32 * (hb0 + th) + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int g = 32 * (gb0 + tg) + 8 * (r >> 2) + 4 * half + (r & 3);
                if (!PAD || (g < nh && h < nh)) part_out[g * nh + h] = acc[tg][th][r];
            }
        }
}

// ---------------------------------------------------------------------------
// fused backward: input gradient and weight-gradient partials in one pass
//
// One read of dY and O serves both gradients: fixed token blocks (a function
// of the shape only), one fp32 weight-gradient partial each, and every
// (token, CH-channel) chunk of dY and O is staged in LDS once.  Three
// configurations split the waves by gradient (BwdCfg::SPLIT): 64 rows with
// CH = 256 on 16 waves, 96 rows with CH = 256 on 12 waves, and 128 rows
// with CH = 128 on 16 waves.  d not a multiple of 256 at 64 rows uses CH =
// 128 on 8 waves with both gradients on every wave; there, with KSET =
// WAVES/4 waves per dW output tile:
//   - dW:  wave w owns output tile w%4 (g-block tile/2, h-block tile%2) over
//          the k-steps t = w/4 (mod KSET); at the end of the block the KSET
//          waves of a tile are added in k-set order (fixed);
//   - dx:  wave w owns M-block w%(CH/32) and N-block w/(CH/32) of the chunk's head mix
//          dX[c, h] = sum_g dY[g, c] W[g, h] (A = dY^T by transposing LDS
//          loads, B = W in registers),
//          rotates paired pe blocks by +phi in registers and writes the
//          results to an LDS output chunk (other pe layouts: an fp32 scratch,
//          rotated in the store phase); the store phase writes dO rows with
//          non-temporal stores.
// The split configurations are described at BwdCfg.  With direct stores
// (DST) their dx waves write their own dO rows to HBM in the compute phase
// and there is no store phase.
// The dx arithmetic (MFMA inputs, k order, rotation expression, tokens per
// tile) is that of the token-part kernel, so dO is bitwise the same as
// postmix_bwd_dx's.  64 head rows (nh <= 32: several tokens per chunk; up to
// 64: padded), 96 or 128 (padded above nh) with pe rotated in registers or
// absent; d a multiple of 128, pe <= 128 (all pe channels in a token's last
// chunk).
// ---------------------------------------------------------------------------

template <int NH, int CH, int WAVES>
struct BwdCfg {
    static constexpr int NT = 64 * WAVES;
    // nh = 128: the waves split by gradient.  Waves 0 .. WAVES/2-1 own two dW
    // tiles each, (g-blocks 2(v/4), 2(v/4)+1; h-block v%4), over every
    // k-step; waves WAVES/2 .. own two dx M-blocks each (2(v/4), 2(v/4)+1;
    // N-block v%4) with their N-block's W fragments in registers.  Both keep
    // 32 registers across the chunk loop (two accumulators, or eight W
    // fragments), in one shared array.  Against one dW tile and one dx block
    // on every wave with W read from LDS per use, the compute phase reads
    // ~40% less LDS.  Only pe rotated in registers.
    // 64 rows on 16 waves split the same way: waves 8 .. 15 each own the two
    // tiles of one h-block (g-blocks 0 and 1) over one of four k-sets, so one
    // O fragment (and one rotated pe operand) serves two MFMAs; waves 0 .. 7
    // each own one dx M-block for both N-blocks, so its transposed dY
    // fragments are read once for two MFMAs, or, with direct dO stores, an
    // M-block pair of one N-block.  Against a tile and a dx block on every
    // wave, the compute phase reads a third less LDS per chunk.
    // 96 rows on 12 waves (one workgroup per CU, 168 registers a wave) split
    // the same way: waves 0 .. 5 each own the three tiles of one h-block
    // (g-blocks 0, 1, 2) over one of two k-sets; waves 6 .. 11 each own four
    // dx M-blocks of one N-block, with its six W fragments in registers.
    static constexpr bool SPLIT = NH == 128 || NH == 96 || (NH == 64 && WAVES == 16);
    static constexpr int NB = NH / 32, KB = NH / 16;
    // SPLIT: g-blocks (dW tiles) per dW wave, dW waves per k-set, k-sets
    // (1 at 128 rows: each tile is one wave's), dx M-blocks per dx wave
    static constexpr int DWG = NB == 3 ? 3 : 2;
    static constexpr int DW_PER_KSET = NB == 3 ? 3 : NB * (NB / 2);
    static constexpr int DW_KSETS = SPLIT ? (WAVES / 2) / DW_PER_KSET : 1;
    // Row pitch (bf16).  The split kernels pad 48 B: rows 12 banks apart (of
    // 64) keep the dW reads (16 rows of 16 B) free of bank conflicts and
    // leave the dx transposed reads (4 rows of 32 + 32 B) 2-way, against
    // 4-way at 16 B of padding (rows 4 banks apart), which measured 2.3x the
    // cost of a conflict-free read.
    static constexpr int PITCH = SPLIT ? CH + 24 : CH + 8;
    // dO rows (no transposed reads).  64 rows split by gradient pad 112 B:
    // the direct dO stores read 8 rows x 128 B per instruction, 1.45x faster
    // there than at 16 B, with the dx result writes (32 rows x 8 B) and the
    // store phase's reads (2 rows x 512 B) as fast as at 16 B
    static constexpr int DPITCH = NH == 64 && SPLIT ? CH + 56 : CH + 8;
    static constexpr int WPITCH = NH + 8;
    static constexpr int VPR = CH / 8;
    static constexpr int VPO = NH * VPR;            // vectors per operand per chunk
    static constexpr int VPT = 2 * VPO / NT;        // vectors (dY + O) per thread per chunk
    static constexpr int OPT = VPO / NT;            // dO vectors per thread per chunk
    static constexpr int KS = CH / 16;              // k-steps of the weight gradient per chunk
    static constexpr int MBC = CH / 32;             // M-blocks of the head mix per chunk
    static constexpr int NTILE = NB * NB;           // dW output tiles
    static constexpr int KSET = WAVES / NTILE;      // waves per dW tile (not SPLIT)
    static constexpr int DXM = SPLIT ? (NB == 2 ? 1 : MBC * NB / (WAVES / 2)) : 1;
    static_assert(SPLIT ? ((WAVES / 2) % DW_PER_KSET == 0 && KS % DW_KSETS == 0 &&
                           (NB == 2 ? MBC == WAVES / 2 : MBC * NB == DXM * (WAVES / 2)) && DXM % (NB == 2 ? 1 : 2) == 0)
                        : ((NH == 64 || NH == 128) && MBC * NB == WAVES && KSET >= 1 && KS % KSET == 0),
                  "fused shape");
    static_assert(VPO % NT == 0, "whole vectors per thread");
    // 96 rows stage W at set-up in the dO buffer (free until the first
    // compute phase), so the chunk buffers at CH = 256 fit the LDS
    static constexpr bool W_IN_DOL = NH == 96;
    // W and the fp32 pe scratch, overlapped (W is consumed at set-up); the
    // scratch is not needed for pe rotated in registers
    __host__ __device__ static size_t aux_bytes(int nope, int pe) {
        const size_t w = W_IN_DOL ? 0 : (size_t)NH * WPITCH * 2;
        const size_t p = pe_pairs_in_blocks(nope, pe) ? 0 : (size_t)NH * (pe + 4) * 4;
        return w > p ? w : p;
    }
    // tokens per group of staged cos/sin rows: whole chunks of tp tokens, at
    // least 16 tokens; at most 32
    __host__ __device__ static int rope_group(int tp) { return tp * ((16 + tp - 1) / tp); }
    static constexpr int RG_MAX = 32;
    // buffers of staged cos/sin groups: two (the next group is fetched while
    // the store phase of the current chunk may still read its rows); one at
    // NH = 96 and 128, whose pe is always rotated in registers, so their
    // store phase reads none
    static constexpr int NBUF = NH >= 96 ? 1 : 2;
    // dY chunk, O chunk, dO chunk, then W / pe scratch, then the buffers of
    // the cos and sin rows of rgt tokens, then (ps) the lo parts of the
    // weight gradient's rotated pe operand, [NH][pe + 8] bf16.  At NH = 128
    // (pe rotated in registers or absent: no pe scratch) the cos/sin rows and
    // the lo parts start where W was: W is only read at set-up, before the
    // first cos/sin rows are fetched.
    static constexpr bool AUX_OVERLAY = NH == 128;
    __host__ __device__ static size_t rope_offset(int nope, int pe) { return AUX_OVERLAY ? 0 : aux_bytes(nope, pe); }
    __host__ __device__ static size_t lds_bytes(int nope, int pe, int rgt, bool ps) {
        const size_t tail = rope_offset(nope, pe) + (size_t)NBUF * rgt * pe * 4 +
                            (ps && pe > 0 ? (size_t)NH * (pe + 8) * 2 : 0);
        const size_t aux = aux_bytes(nope, pe);
        return (size_t)2 * NH * PITCH * 2 + (size_t)NH * DPITCH * 2 + (tail > aux ? tail : aux);
    }
};

template <int NH, int CH, int WAVES, bool PAD, bool PS, bool DST>
__global__ __launch_bounds__(64 * WAVES, WAVES == 12 ? 3 : 4) void bwd_fused_kernel(
    const uint16_t* __restrict__ dY, const uint16_t* __restrict__ O, const uint16_t* __restrict__ W,
    const float* __restrict__ rcos, const float* __restrict__ rsin, int64_t table_rows,
    const int32_t* __restrict__ positions, int64_t sq, int nh, int nope, int pe,
    uint16_t* __restrict__ dO, float* __restrict__ partials, int64_t ngroups, int ptok, int rgt, int spans) {
    // PAD: nh < NH.  A chunk then holds ptok consecutive tokens (ptok*nh
    // consecutive rows of the [sq*nh, d] arrays; W staged block-diagonally,
    // one copy per token, exactly as in the token-part kernel), the other rows
    // are zero padding (never loaded or stored), and the partial is the sum of
    // the ptok diagonal [nh, nh] blocks.  Otherwise nh == NH and ptok == 1.
    using C = BwdCfg<NH, CH, WAVES>;
    const int tp = PAD ? ptok : 1;
    // rgt: tokens per staged group of cos/sin rows, a multiple of tp
    // PS: the weight gradient's rotated pe operand is formed once per chunk
    // (hi in place of the staged O, lo in lol) instead of in each k-step
    // that reads it, i.e. by every wave of the tile's row block
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    uint16_t* dyl = smem;                               // [NH][PITCH]
    uint16_t* ol = dyl + NH * C::PITCH;                 // [NH][PITCH]
    uint16_t* dol = ol + NH * C::PITCH;                 // [NH][DPITCH]
    uint16_t* const auxp = dol + NH * C::DPITCH;
    uint16_t* wl = C::W_IN_DOL ? dol : auxp;            // [NH][WPITCH] bf16 at set-up
    float* pes = reinterpret_cast<float*>(auxp);        // [NH][pe + 4] fp32, after set-up
    const int pes_pitch = pe + 4;
    // two buffers of the cos/sin rows of rgt consecutive tokens: [2][rgt][pe]
    // floats (cos then sin each); consecutive groups alternate
    float* const rope_g = reinterpret_cast<float*>(reinterpret_cast<char*>(auxp) + C::rope_offset(nope, pe));

    const int d = nope + pe, h2 = pe >> 1;
    const int lpitch = pe + 8;
    const int cpt = d / CH;
    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, Q = half;
    // the wave index in a scalar register frees the vector registers of its
    // derived indices (tile, k-set, blocks), which otherwise spill
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tile = wave % C::NTILE, kset = wave / C::NTILE;
    // SPLIT: dw_role waves own dW tiles (gb + j, hb), j < DWG, over k-set
    // dkset; the others dx M-blocks mb .. mb + DXM - 1 of N-block nb (96 and
    // 128 rows) or M-block mb of both N-blocks (64 rows)
    // (at 64 rows the dx waves take the lower wave indices: the dx waves set
    // the compute phase's length, and lower waves win the arbitration for the
    // MFMA and LDS pipes; at 128 rows that order measured slower)
    const bool dw_role = !C::SPLIT || (C::NB == 2 ? wave >= WAVES / 2 : wave < WAVES / 2);
    const int vs = wave % (WAVES / 2);
    const int gb = C::SPLIT ? 2 * ((vs / C::NB) % (C::NB / 2)) : tile / C::NB;
    const int hb = C::SPLIT ? vs % C::NB : tile % C::NB;
    const int dkset = C::SPLIT ? vs / C::DW_PER_KSET : 0;
    // DST: the dx waves store their own dO rows (below); at 64 rows they
    // then own M-block pairs (mb, mb + 1) of one N-block
    static_assert(!DST || C::SPLIT, "direct dO stores: waves split by gradient");
    constexpr int DXW = C::NB == 2 ? 2 : C::DXM;  // DST: M-blocks per dx wave
    const int mb = C::SPLIT ? (C::NB == 2 ? (DST ? 2 * (vs >> 1) : vs) : C::DXM * (vs / C::NB)) : wave % C::MBC;
    const int nb = C::SPLIT ? (C::NB == 2 ? (DST ? (vs & 1) : 0) : vs % C::NB) : wave / C::MBC;
    // offsets into a chunk's cos/sin rows of the tokens of this lane's dW row
    // (32*hb + lane%32) and dx row (32*nbx + lane%32); padding rows take any
    // staged token's
    const int ph = PAD ? (32 * hb + (lane & 31)) / nh : 0;
    const int ph_off = (ph < tp ? ph : tp - 1) * pe;
    auto pr_off_of = [&](int nbx) {
        const int pr = PAD ? (32 * nbx + (lane & 31)) / nh : 0;
        return (pr < tp ? pr : tp - 1) * pe;
    };

    // token block tb of B = gridDim.x / spans holds the token groups (tp
    // tokens each, one chunk's rows) [tb*G/B, (tb+1)*G/B) of the G = ngroups
    // groups; channel span y = b % spans takes the CH-channel parts
    // [y*cpt/spans, (y+1)*cpt/spans) of each (spans > 1 only for very wide
    // rows, to bound the weight gradient's accumulation chain).  One partial
    // per workgroup.
    const int64_t nbt = gridDim.x / spans, tb = blockIdx.x / spans;
    const int y = (int)(blockIdx.x - tb * spans);
    const int64_t s_begin = tb * ngroups / nbt * tp;
    int64_t s_end = (tb + 1) * ngroups / nbt * tp;
    if (s_end > sq) s_end = sq;
    const int p0 = (int)((int64_t)y * cpt / spans), cps = (int)((int64_t)(y + 1) * cpt / spans) - p0;
    // At 96 and 128 rows token block tb takes the groups tb, tb + B, tb + 2B,
    // ... instead (about the same count), so the blocks running at once work
    // on neighbouring tokens: nh = 128, sq = 8192 585 -> 569 us settled
    // (621 -> 618 in the benchmark's regime), nh = 96 460 -> 456 us.  At 64
    // rows contiguous ranges measured faster (517 against 523 us settled).
    constexpr bool kStridedTokens = NH >= 96;
    const int ngr = kStridedTokens ? (tb < ngroups ? (int)((ngroups - 1 - tb) / nbt + 1) : 0)
                                   : (int)((s_end - s_begin + tp - 1) / tp);
    auto group_tok = [&](int j) -> int64_t {  // first token of the block's j-th group
        return kStridedTokens ? (tb + nbt * (int64_t)j) * tp : s_begin + (int64_t)j * tp;
    };
    const int64_t s_lim = kStridedTokens ? sq : s_end;  // tokens of a group end below this
    const int nchunks = ngr * cps;

    u32x4 v[C::VPT];
    // cos and sin rows of the rgt tokens of groups j0, j0 + 1, .. of the
    // block -> LDS buffer `buf`; read once per rgt tokens instead of once per
    // chunk.  Rows past the last token are zeros: the padding rows of a
    // partial chunk rotate zeros with them, and their products must stay
    // exact zeros.
    auto load_rope_group = [&](int j0, int buf) {
        float* const rg = rope_g + (C::NBUF == 2 ? buf : 0) * rgt * pe;
        const int q4 = pe >> 2, half4 = pe >> 3;  // f32x4 per token row (cos + sin), per table row
        for (int idx = tid; idx < rgt * q4; idx += C::NT) {
            const int t = idx / q4, q = idx - t * q4;
            const int jt = j0 + t / tp;                 // the row's group
            const int64_t st = group_tok(jt) + t % tp;  // and token
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            if (jt < ngr && st < s_lim) {
                const int64_t prow = table_row(positions, st, table_rows);
                const float* tab = q < half4 ? rcos : rsin;
                const int qq = q < half4 ? q : q - half4;
                x = reinterpret_cast<const f32x4*>(tab + prow * h2)[qq];
            }
            reinterpret_cast<f32x4*>(rg + t * pe)[q] = x;
        }
    };
    // head rows of chunk k backed by tokens below s_lim
    auto chunk_rows = [&](int k) -> int {
        if (!PAD) return NH;
        const int64_t left = s_lim - group_tok(k / cps);
        return (int)(left < tp ? left : tp) * nh;
    };
    // The loads are unconditional: padding rows re-read the chunk's last row
    // (an L2 hit) and are zeroed when staged.  Exec-masked loads would need
    // their addresses live across the loop, and a spill reload there waits
    // for every load in flight (scratch and global loads share one counter),
    // which serialises the prefetch.  In-chunk offsets fit 32 bits (d <= 2^24).
    auto load_chunk = [&](int k) {
        const int64_t s = group_tok(k / cps);  // first token of the chunk
        const int part = p0 + k % cps;
        const int rows = chunk_rows(k);
        const int64_t rowbase = s * nh * (int64_t)d + part * CH;
        const uint16_t* const dyb = dY + rowbase;
        const uint16_t* const ob = O + rowbase;
        // 96 rows: the thread index is made opaque here, so the per-vector
        // offsets are recomputed per chunk (a few adds) instead of kept across
        // the chunk loop, where eight 64-bit offsets were spilled and their
        // reloads serialised the prefetch
        int lt = tid;
        if (C::W_IN_DOL) asm volatile("" : "+v"(lt));
#pragma unroll
        for (int j = 0; j < C::VPT; ++j) {
            const int q = j * C::NT + lt;
            const int op = q / C::VPO;               // 0: dY, 1: O (compile-time per j)
            const int rem = q % C::VPO;
            int row = rem / C::VPR;
            const int c8 = rem % C::VPR;
            if (PAD) row = row < rows ? row : rows - 1;
            const uint32_t off = (uint32_t)row * (uint32_t)d + 8u * (uint32_t)c8;
            v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>((op == 0 ? dyb : ob) + off));
        }
    };
    auto stage_chunk = [&](int k) {  // registers of chunk k -> LDS (padding rows as zeros)
        const int rows = chunk_rows(k);
        int lt = tid;  // opaque at 96 rows, as in load_chunk
        if (C::W_IN_DOL) asm volatile("" : "+v"(lt));
#pragma unroll
        for (int j = 0; j < C::VPT; ++j) {
            const int q = j * C::NT + lt;
            const int op = q / C::VPO;
            const int rem = q % C::VPO;
            const int row = rem / C::VPR, c8 = rem % C::VPR;
            const u32x4 x = (!PAD || row < rows) ? v[j] : u32x4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>((op == 0 ? dyl : ol) + row * C::PITCH + 8 * c8) = x;
        }
    };
    if (nchunks > 0) load_chunk(0);
    if (!C::AUX_OVERLAY && pe > 0 && nchunks > 0) load_rope_group(0, 0);

    // W -> LDS -> this wave's dx B operand (B[k=g][n=h] = W[g][h], N-block nb).
    // SPLIT stages W transposed, [h][g]: a lane's B fragment (column h, 8
    // consecutive g) is then one 16-byte read.
    if (C::SPLIT) {
        for (int q = tid; q < NH * NH; q += C::NT) {
            const int row = q / NH, col = q % NH;  // W[row][col] -> wl[col][row]
            const int p = row / nh, pc = col / nh;
            uint16_t w = 0;
            if (!PAD) w = W[q];
            else if (p == pc && p < tp) w = W[(row - p * nh) * nh + (col - p * nh)];
            wl[col * C::WPITCH + row] = w;
        }
    } else if (!PAD) {
        for (int q = tid; q < NH * NH / 8; q += C::NT) {
            const int row = q / (NH / 8), c8 = q % (NH / 8);
            *reinterpret_cast<u32x4*>(wl + row * C::WPITCH + 8 * c8) = reinterpret_cast<const u32x4*>(W)[q];
        }
    } else {  // block-diagonal: W at rows and columns p*nh .. p*nh+nh-1 for p < tp, zeros elsewhere
        for (int q = tid; q < NH * NH; q += C::NT) {
            const int row = q / NH, col = q % NH;
            const int p = row / nh, pc = col / nh;
            wl[row * C::WPITCH + col] =
                (p == pc && p < tp) ? W[(row - p * nh) * nh + (col - p * nh)] : (uint16_t)0;
        }
    }
    __syncthreads();
    bf16x8 wf[C::SPLIT ? 1 : C::KB];  // W fragments in registers (not SPLIT)
    // SPLIT: a dW wave's DWG accumulators, or a dx wave's W fragments (eight;
    // six at 96 rows; fragment kb in keep[kb / 4], elements 4(kb % 4) ..)
    f32x16 keep[C::DWG];
#pragma unroll
    for (int j = 0; j < C::DWG; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) keep[j][r] = 0.0f;
    if (!C::SPLIT) {
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) wf[kb] = tr_frag(wl + (16 * kb) * C::WPITCH + 32 * nb, C::WPITCH, lane);
    } else if (!dw_role) {
        // 96 and 128 rows: the six or eight fragments of N-block nb (fragment
        // kb in keep[kb / 4]); 64 rows: the four of each N-block (N-block n in keep[n])
#pragma unroll
        for (int kb = 0; kb < (C::NB == 2 && !DST ? 8 : C::KB); ++kb) {
            const int n = C::NB == 2 && !DST ? kb >> 2 : nb, k = C::NB == 2 && !DST ? kb & 3 : kb;
            const u32x4 f = *reinterpret_cast<const u32x4*>(wl + (32 * n + (lane & 31)) * C::WPITCH + 16 * k +
                                                            8 * (lane >> 5));
#pragma unroll
            for (int e = 0; e < 4; ++e) keep[kb >> 2][4 * (kb & 3) + e] = __uint_as_float(f[e]);
        }
    }
    __syncthreads();  // W's LDS becomes the pe scratch (or the cos/sin rows, or dO)
    if (C::AUX_OVERLAY && pe > 0 && nchunks > 0) load_rope_group(0, 0);

    f32x16 acc_w;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_w[r] = 0.0f;

    // Pipeline: chunk k is computed from the dY/O buffers; once every wave is
    // done with them (barrier), chunk k+1 (already in registers) is staged
    // there and chunk k+2 is requested, and only then are chunk k's dO rows
    // stored (they live in separate buffers).  Two barriers per chunk.
    // ---- PS: the rotated pe operand of chunk kk, once per chunk.  A task is
    // a row and 4 channels i .. i+3 of the first half with their partners
    // i+h2 ..: both halves are read and written by the same thread (4
    // channels, not 8: this pass sets the kernel's register peak).  hi goes in
    // place of the staged O, lo to lol.  It runs in the staging phase, right
    // after the next chunk's loads are issued (the memory wait hides it), by
    // every wave, instead of in the compute phase, where the dW waves set the
    // pace.  Each row takes the cos/sin row of its token (one token per chunk
    // at 128 rows).  vh (tasks per row) is a power of two (checked at launch):
    // a shift and a mask split the task index.  A division there made the
    // compiler keep a 64-bit value across the chunk loop, spilled, and its
    // reload waited for the chunk prefetch (nh = 96: 65 us of 760).
    auto chunk_has_pe = [&](int kk) { return pe > 0 && (p0 + kk % cps) * CH + CH > nope; };
    auto pe_pass = [&](int kk) {
        static_assert(!PS || C::SPLIT, "the pe pass is compiled for waves split by gradient only");
        const int c_base = (p0 + kk % cps) * CH;
        const int tok = (kk / cps) * tp;
        const float* csl = rope_g + ((C::NBUF == 2 ? (tok / rgt) & 1 : 0) * rgt + tok % rgt) * pe;
        uint16_t* const lol = reinterpret_cast<uint16_t*>(rope_g + C::NBUF * rgt * pe);  // [NH][pe + 8]
        const int L0 = nope - c_base;  // local first pe channel (the whole pe range is in this chunk)
        const int vh = h2 >> 2;
        const int lvh = __builtin_ctz((unsigned)vh);
        for (int task = tid; task < (NH << lvh); task += C::NT) {
            const int row = task >> lvh, i = 4 * (task & (vh - 1));
            uint16_t* const o1 = ol + row * C::PITCH + L0 + i;
            uint16_t* const o2 = o1 + h2;
            const uint2 a = *reinterpret_cast<const uint2*>(o1), b = *reinterpret_cast<const uint2*>(o2);
            int rt = PAD && NH == 64 ? row / nh : 0;  // the row's token (padding rows: any staged one)
            rt = rt < tp ? rt : tp - 1;
            const float* cr = csl + rt * pe + i;
            const f32x4 c4 = *reinterpret_cast<const f32x4*>(cr), s4 = *reinterpret_cast<const f32x4*>(cr + h2);
            float cs[4], sp[4], sm[4];
            uint32_t aw[2] = {a.x, a.y}, bw[2] = {b.x, b.y}, h1[2], l1[2], hh2[2], ll2[2];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                cs[e] = c4[e];
                sp[e] = s4[e];
                sm[e] = -s4[e];
            }
            rotate_split<2>(aw, bw, cs, sp, h1, l1);   // first half: a C + b S
            rotate_split<2>(bw, aw, cs, sm, hh2, ll2);  // second half: b C - a S
            *reinterpret_cast<uint2*>(o1) = uint2{h1[0], h1[1]};
            *reinterpret_cast<uint2*>(o2) = uint2{hh2[0], hh2[1]};
            *reinterpret_cast<uint2*>(lol + row * lpitch + i) = uint2{l1[0], l1[1]};
            *reinterpret_cast<uint2*>(lol + row * lpitch + h2 + i) = uint2{ll2[0], ll2[1]};
        }
    };

    if (nchunks > 0) {
        stage_chunk(0);
        if (nchunks > 1) load_chunk(1);
    }
    __syncthreads();
    if (PS && nchunks > 0 && chunk_has_pe(0)) {
        pe_pass(0);
        __syncthreads();
    }
    for (int k = 0; k < nchunks; ++k) {
        const int64_t s = group_tok(k / cps);  // first token of the chunk
        const int part = p0 + k % cps;
        const int c_base = part * CH;
        const bool chunk_pe = pe > 0 && c_base + CH > nope;
        // cos/sin rows of the chunk's first token; a row r of the chunk uses those of token r / nh
        const int tok = (k / cps) * tp;  // the chunk's first token within the block
        const float* csl = rope_g + ((C::NBUF == 2 ? (tok / rgt) & 1 : 0) * rgt + tok % rgt) * pe;
        const float* snl = csl + (pe >> 1);
        uint16_t* const lol = reinterpret_cast<uint16_t*>(rope_g + C::NBUF * rgt * pe);  // [NH][pe + 8]

        // the weight gradient's B operand of a pe k-step: the rotated O rows
        // (h, channels c .. c+7), split into hi + lo; PS: hi formed in place
        // of O, lo beside it
        auto pe_operand = [&](int c, int cg, int h, const u32x4& own, u32x4& hi_out, u32x4& lo_out) {
            if (PS) {
                u32x4 lo = {0u, 0u, 0u, 0u};
                if (cg >= nope) lo = *reinterpret_cast<const u32x4*>(lol + h * lpitch + (cg - nope));
                hi_out = own;
                lo_out = lo;
                return;
            }
                u32x4 hi = own, lo = {0u, 0u, 0u, 0u};
            if (cg >= nope) {
                const bool first = cg < nope + h2;
                const int i0 = first ? cg - nope : cg - nope - h2;
                const float sgn = first ? 1.0f : -1.0f;
                const float* cr = csl + ph_off + i0;
                const float* sr = snl + ph_off + i0;
                const u32x4 par = *reinterpret_cast<const u32x4*>(ol + h * C::PITCH + (first ? c + h2 : c - h2));
                const f32x4 c0 = *reinterpret_cast<const f32x4*>(cr), c1 = *reinterpret_cast<const f32x4*>(cr + 4);
                const f32x4 s0 = *reinterpret_cast<const f32x4*>(sr), s1 = *reinterpret_cast<const f32x4*>(sr + 4);
                float cs[8], sn[8];
                uint32_t ow[4], pw[4], hw[4], lw[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    cs[e] = c0[e]; cs[4 + e] = c1[e];
                    sn[e] = sgn * s0[e]; sn[4 + e] = sgn * s1[e];
                    ow[e] = own[e]; pw[e] = par[e];
                }
                rotate_split8(ow, pw, cs, sn, hw, lw);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) { hi[jj] = hw[jj]; lo[jj] = lw[jj]; }
            }
            hi_out = hi;
            lo_out = lo;
        };

        if (C::SPLIT && dw_role) {
            // ---- weight gradient: tiles (gb + j, hb), j < DWG, k-steps
            // t = dkset, dkset + DW_KSETS, ... (every k-step at 128 rows).
            // The lane's channel offset is made opaque per chunk: otherwise
            // the compiler keeps one precomputed offset per k-step live across
            // the chunk loop, they spill, and their reloads in the pe k-steps
            // wait for the chunk prefetch (scratch and global loads share a
            // counter).  Recomputing an offset is one add.
            int h8 = 8 * half;
            asm volatile("" : "+v"(h8));
#pragma unroll
            for (int j = 0; j < C::KS / C::DW_KSETS; ++j) {
                const int t = dkset + C::DW_KSETS * j;
                const int c = 16 * t + h8;
                bf16x8 a[C::DWG];
#pragma unroll
                for (int g = 0; g < C::DWG; ++g)
                    a[g] = *reinterpret_cast<const bf16x8*>(dyl + (32 * (gb + g) + (lane & 31)) * C::PITCH + c);
                const int h = 32 * hb + (lane & 31);
                const u32x4 own = *reinterpret_cast<const u32x4*>(ol + h * C::PITCH + c);
                const bool step_pe = chunk_pe && c_base + 16 * t + 16 > nope;  // wave-uniform
                // the branches only form operands: MFMAs under a branch gave
                // each accumulator a second register copy at the join
                u32x4 hi = own, lo = {0u, 0u, 0u, 0u};
                if (step_pe) pe_operand(c, c_base + c, h, own, hi, lo);
#pragma unroll
                for (int g = 0; g < C::DWG; ++g) {
                    keep[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[g], as_bf16x8(hi), keep[g], 0, 0, 0);
                    if (step_pe) keep[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[g], as_bf16x8(lo), keep[g], 0, 0, 0);
                }
            }
        } else if (!C::SPLIT) {
            // ---- weight gradient: tile (gb, hb), k-steps t = kset, kset + KSET, ...
#pragma unroll
            for (int j = 0; j < C::KS / C::KSET; ++j) {
                const int t = kset + C::KSET * j;
                const int c = 16 * t + 8 * half;
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(dyl + (32 * gb + (lane & 31)) * C::PITCH + c);
                const int h = 32 * hb + (lane & 31);
                const u32x4 own = *reinterpret_cast<const u32x4*>(ol + h * C::PITCH + c);
                const bool step_pe = chunk_pe && c_base + 16 * t + 16 > nope;  // wave-uniform
                if (!step_pe) {
                    acc_w = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16x8(own), acc_w, 0, 0, 0);
                } else {
                    u32x4 hi, lo;
                    pe_operand(c, c_base + c, h, own, hi, lo);
                    acc_w = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16x8(hi), acc_w, 0, 0, 0);
                    acc_w = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16x8(lo), acc_w, 0, 0, 0);
                }
            }
        }

        // ---- input gradient: M-block m (channels), N-block n (heads); bfrag(kb)
        // gives the lane's W fragment of k-block kb
        const bool paired = chunk_pe && pe_pairs_in_blocks(nope, pe);
        const int L = nope - c_base;  // local index of the first pe channel (chunks with pe)
        // the results of block (m, n): paired pe blocks rotated in registers,
        // other pe channels to the fp32 scratch, nope channels rounded to bf16
        auto dx_store = [&](const f32x16& acc, int m, int n) {
            const bool pb = paired && 32 * m >= L;  // a paired pe block (wave-uniform)
            const int q = m - (L >> 5);
            const int hrow = 32 * n + (lane & 31);
            if (pb) {
                const int pr_off = pr_off_of(n);
                rotate_paired_block(acc, dol, C::DPITCH, hrow, L, h2, q, Q, csl + pr_off, snl + pr_off, -1.0f);
            }
#pragma unroll
            for (int a = 0; a < 4 && !pb; ++a) {
                const int cl = 32 * m + 8 * a + 4 * Q;
                const int cg = c_base + cl;
                if (cg < nope) {
                    uint2 o;
                    o.x = pack_bf16(acc[4 * a], acc[4 * a + 1]);
                    o.y = pack_bf16(acc[4 * a + 2], acc[4 * a + 3]);
                    *reinterpret_cast<uint2*>(dol + hrow * C::DPITCH + cl) = o;
                } else {
                    f32x4 o = {acc[4 * a], acc[4 * a + 1], acc[4 * a + 2], acc[4 * a + 3]};
                    *reinterpret_cast<f32x4*>(pes + hrow * pes_pitch + (cg - nope)) = o;
                }
            }
        };
        // the lane's A fragment columns of M-block m (a paired pe block takes
        // 16 first-half channels and their 16 partners)
        auto a_cols = [&](int m, int& clo, int& chi) {
            const bool pb = paired && 32 * m >= L;
            const int q = m - (L >> 5);
            clo = pb ? L + 16 * q : 32 * m;
            chi = pb ? L + h2 + 16 * q : 32 * m + 16;
        };
        auto dx_block = [&](int m, auto&& bfrag) {
            f32x16 acc;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
            int clo, chi;
            a_cols(m, clo, chi);
            if constexpr (C::SPLIT) {  // A fragments one k-block ahead (registers)
                bf16x8 a = tr_frag2(dyl, clo, chi, C::PITCH, lane);
#pragma unroll
                for (int kb = 0; kb < C::KB; ++kb) {
                    const bf16x8 an = tr_frag2(dyl + (16 * (kb + 1 < C::KB ? kb + 1 : kb)) * C::PITCH, clo, chi,
                                               C::PITCH, lane);
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bfrag(kb), acc, 0, 0, 0);
                    a = an;
                }
            } else {
                bf16x8 af[C::KB];
#pragma unroll
                for (int kb = 0; kb < C::KB; ++kb)
                    af[kb] = tr_frag2(dyl + (16 * kb) * C::PITCH, clo, chi, C::PITCH, lane);
#pragma unroll
                for (int kb = 0; kb < C::KB; ++kb)
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kb], bfrag(kb), acc, 0, 0, 0);
            }
            dx_store(acc, m, nb);
        };
        auto kept = [&](int kb) {
            u32x4 f;
#pragma unroll
            for (int e = 0; e < 4; ++e) f[e] = __float_as_uint(keep[kb >> 2][4 * (kb & 3) + e]);
            return as_bf16x8(f);
        };
        // DST: this dx wave's own dO rows (32 rows of N-block nb x the 32*DXW
        // channels of its M-blocks: whole lines that no other wave writes)
        // from its dO buffer columns to HBM, here in the compute phase, where
        // the dx waves would otherwise wait for the dW waves; no store phase.
        // Each lane reads back what lanes of this wave wrote: LDS accesses of
        // one wave complete in order, and the fences keep the compiler from
        // moving them.
        auto store_own_dO = [&]() {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            constexpr int LPR = 4 * DXW, RPI = 64 / LPR;  // lanes per row, rows per instruction
            const int rows_k = chunk_rows(k);
            uint16_t* const outs = dO + s * nh * (int64_t)d + c_base;
            int ln = lane;  // opaque at 96 rows, as in load_chunk
            if (C::W_IN_DOL) asm volatile("" : "+v"(ln));
#pragma unroll
            for (int j = 0; j < 32 / RPI; ++j) {
                const int row = 32 * nb + RPI * j + ln / LPR, cl = 32 * mb + 8 * (ln % LPR);
                if (PAD && row >= rows_k) continue;  // padding rows
                const u32x4 o = *reinterpret_cast<const u32x4*>(dol + row * C::DPITCH + cl);
                __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(outs + row * (int64_t)d + cl));
            }
        };
        if (!C::SPLIT) {
            dx_block(mb, [&](int kb) { return wf[C::SPLIT ? 0 : kb]; });
        } else if (!dw_role && C::NB == 2 && DST) {
            // 64 rows, direct stores: M-blocks mb, mb + 1 of N-block nb
            dx_block(mb, kept);
            dx_block(mb + 1, kept);
            store_own_dO();
        } else if (!dw_role && C::NB == 2) {
            // 64 rows: M-block mb for both N-blocks from one read of its A
            // fragments; each block's MFMA inputs and k order are the
            // token-part kernel's, so dO keeps its bits
            int clo, chi;
            a_cols(mb, clo, chi);
            bf16x8 af[C::KB];
#pragma unroll
            for (int kb = 0; kb < C::KB; ++kb) af[kb] = tr_frag2(dyl + (16 * kb) * C::PITCH, clo, chi, C::PITCH, lane);
            f32x16 acc0, acc1;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc0[r] = acc1[r] = 0.0f;
#pragma unroll
            for (int kb = 0; kb < C::KB; ++kb) {
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kb], kept(kb), acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kb], kept(4 + kb), acc1, 0, 0, 0);
            }
            dx_store(acc0, mb, 0);
            dx_store(acc1, mb, 1);
        } else if (!dw_role && C::NB == 3) {
            // 96 rows: the next M-block's six A fragments are read while this
            // block's MFMAs run (the registers allow it at 12 waves); one
            // fragment ahead left the dx waves waiting on LDS latency in each
            // k-step.  MFMA inputs and k order are those of dx_block.
            bf16x8 af[C::KB], an[C::KB];
            auto read_frags = [&](int m, bf16x8* f) {
                int clo, chi;
                a_cols(m, clo, chi);
#pragma unroll
                for (int kb = 0; kb < C::KB; ++kb) f[kb] = tr_frag2(dyl + (16 * kb) * C::PITCH, clo, chi, C::PITCH, lane);
            };
            read_frags(mb, af);
#pragma unroll
            for (int i = 0; i < C::DXM; ++i) {
                if (i + 1 < C::DXM) read_frags(mb + i + 1, an);
                f32x16 acc;
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
                for (int kb = 0; kb < C::KB; ++kb) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kb], kept(kb), acc, 0, 0, 0);
                dx_store(acc, mb + i, nb);
#pragma unroll
                for (int kb = 0; kb < C::KB; ++kb) af[kb] = an[kb];
            }
            if (DST) store_own_dO();
        } else if (!dw_role) {
#pragma unroll
            for (int i = 0; i < C::DXM; ++i) dx_block(mb + i, kept);
            if (DST) store_own_dO();
        }
        __syncthreads();  // dY/O buffers free; dO and the pe scratch complete
        if (k + 1 < nchunks) {
            // a new group of cos/sin rows goes to the other buffer (the one of
            // the group before this chunk's), ahead of the chunk prefetch, so
            // waiting for the table rows waits for nothing else in flight
            // but chunk k+1, which the staging needs anyway
            const int tok1 = ((k + 1) / cps) * tp;
            if (pe > 0 && (k + 1) % cps == 0 && tok1 % rgt == 0) load_rope_group(tok1 / tp, (tok1 / rgt) & 1);
            stage_chunk(k + 1);
            if (k + 2 < nchunks) load_chunk(k + 2);  // in flight during two compute phases
            if (PS && chunk_has_pe(k + 1)) {
                __syncthreads();  // chunk k+1 staged by every thread
                pe_pass(k + 1);   // visible to its compute phase after the barrier below
            }
        }

        // ---- dO rows of the chunk; pe pairs turned by +phi (DST: stored by
        // the dx waves in the compute phase)
        uint16_t* outs = dO + s * nh * (int64_t)d + c_base;
        const int rows_k = chunk_rows(k);
        int lt = tid;  // opaque at 96 rows, as in load_chunk
        if (C::W_IN_DOL) asm volatile("" : "+v"(lt));
#pragma unroll
        for (int j = 0; j < (DST ? 0 : C::OPT); ++j) {
            const int q = j * C::NT + lt;
            const int row = q / C::VPR, c8 = q % C::VPR;
            if (PAD && row >= rows_k) continue;  // padding rows
            const int cl = 8 * c8, cg = c_base + cl;
            u32x4 o;
            if (cg < nope || paired) {
                o = *reinterpret_cast<const u32x4*>(dol + row * C::DPITCH + cl);
            } else {
                const int i = cg - nope;
                const bool first = i < h2;
                const int ii = first ? i : i - h2;
                const float* own = pes + row * pes_pitch + i;
                const float* par = pes + row * pes_pitch + (first ? i + h2 : i - h2);
                const int rp = PAD ? (row / nh) * pe : 0;  // the row's token's cos/sin
                const f32x4 o0 = reinterpret_cast<const f32x4*>(own)[0], o1 = reinterpret_cast<const f32x4*>(own)[1];
                const f32x4 p0 = reinterpret_cast<const f32x4*>(par)[0], p1 = reinterpret_cast<const f32x4*>(par)[1];
                const f32x4 c0 = reinterpret_cast<const f32x4*>(csl + rp + ii)[0];
                const f32x4 c1 = reinterpret_cast<const f32x4*>(csl + rp + ii)[1];
                const f32x4 s0 = reinterpret_cast<const f32x4*>(snl + rp + ii)[0];
                const f32x4 s1 = reinterpret_cast<const f32x4*>(snl + rp + ii)[1];
                // +phi: first half a C - b S, second half b C + a S
                const float sg = first ? -1.0f : 1.0f;
                float y[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    y[e] = o0[e] * c0[e] + sg * (p0[e] * s0[e]);
                    y[4 + e] = o1[e] * c1[e] + sg * (p1[e] * s1[e]);
                }
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) o[jj] = pack_bf16(y[2 * jj], y[2 * jj + 1]);
            }
            __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(outs + row * (int64_t)d + cl));
        }
        __syncthreads();  // dO buffers read; chunk k+1 and its cos/sin rows staged
    }

    // ---- dW partial: the k-sets of each tile summed in k-set order (fixed);
    // SPLIT: each wave owns DWG tiles over its k-set (at 128 rows every k-step)
    float* red = reinterpret_cast<float*>(smem);
    constexpr int NPAIR = C::DW_PER_KSET;  // SPLIT: dW waves of one k-set
    const int pair = vs % NPAIR;
    auto red_slot = [&](int k, int j, int r) -> float& {
        return red[((((k - 1) * NPAIR + pair) * C::DWG + j) * 16 + r) * 64 + lane];
    };
    // LDS left for the reduction and the partial (chunk buffers and dO)
    constexpr int RED_LDS = 2 * NH * C::PITCH * 2 + NH * C::DPITCH * 2;
    if (!C::SPLIT && kset != 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) red[(((kset - 1) * C::NTILE + tile) * 16 + r) * 64 + lane] = acc_w[r];
    }
    if (C::SPLIT && C::DW_KSETS > 1 && dw_role && dkset != 0) {
#pragma unroll
        for (int j = 0; j < C::DWG; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) red_slot(dkset, j, r) = keep[j][r];
    }
    __syncthreads();
    if constexpr (C::SPLIT) {
        const bool owner = dw_role && dkset == 0;
        if (C::DW_KSETS > 1 && owner) {
#pragma unroll
            for (int k = 1; k < C::DW_KSETS; ++k)
#pragma unroll
                for (int j = 0; j < C::DWG; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) keep[j][r] += red_slot(k, j, r);
        }
        if constexpr (PAD) {
            // the [NH, NH] tile sums to LDS (after the k-set area), then the
            // partial is the sum of the tp diagonal [nh, nh] blocks, p = 0, 1,
            // .. in order (tp = 1 at 128 rows: the block itself)
            constexpr int RED = (C::DW_KSETS - 1) * NPAIR * C::DWG * 16 * 64;
            static_assert((RED + NH * (NH + 1)) * 4 <= RED_LDS, "partial area");
            float* m = red + RED;
            if (owner) {
#pragma unroll
                for (int j = 0; j < C::DWG; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        m[(32 * (gb + j) + 8 * (r >> 2) + 4 * half + (r & 3)) * (NH + 1) + 32 * hb + (lane & 31)] =
                            keep[j][r];
            }
            __syncthreads();
            float* part_out = partials + (int64_t)blockIdx.x * nh * nh;
            for (int idx = tid; idx < nh * nh; idx += C::NT) {
                const int g = idx / nh, h = idx - g * nh;
                float sum = m[g * (NH + 1) + h];
                for (int p = 1; p < tp; ++p) sum += m[(p * nh + g) * (NH + 1) + p * nh + h];
                part_out[idx] = sum;
            }
            return;
        } else {
            if (!owner) return;
            float* part_out = partials + (int64_t)blockIdx.x * nh * nh;
            const int h = 32 * hb + (lane & 31);
#pragma unroll
            for (int j = 0; j < C::DWG; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    part_out[(32 * (gb + j) + 8 * (r >> 2) + 4 * half + (r & 3)) * nh + h] = keep[j][r];
            return;
        }
    } else if constexpr (PAD) {
        // the full [NH, NH] sum goes to LDS (after the k-set area), then the
        // partial is the sum of the tp diagonal [nh, nh] blocks, p = 0, 1, ..
        // in order (tp = 1: the block itself)
        constexpr int RED = (C::KSET - 1) * C::NTILE * 16 * 64;  // floats of the k-set area
        static_assert((RED + NH * (NH + 1)) * 4 <= RED_LDS, "diagonal-block area");
        float* m = red + RED;
        if (kset == 0) {
#pragma unroll
            for (int k = 1; k < C::KSET; ++k)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc_w[r] += red[(((k - 1) * C::NTILE + tile) * 16 + r) * 64 + lane];
#pragma unroll
            for (int r = 0; r < 16; ++r)
                m[(32 * gb + 8 * (r >> 2) + 4 * half + (r & 3)) * (NH + 1) + 32 * hb + (lane & 31)] = acc_w[r];
        }
        __syncthreads();
        float* part_out = partials + (int64_t)blockIdx.x * nh * nh;
        for (int idx = tid; idx < nh * nh; idx += C::NT) {
            const int g = idx / nh, h = idx - g * nh;
            float sum = m[g * (NH + 1) + h];
            for (int p = 1; p < tp; ++p) sum += m[(p * nh + g) * (NH + 1) + p * nh + h];
            part_out[idx] = sum;
        }
        return;
    }
    if (kset != 0) return;
#pragma unroll
    for (int k = 1; k < C::KSET; ++k)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_w[r] += red[(((k - 1) * C::NTILE + tile) * 16 + r) * 64 + lane];
    float* part_out = partials + (int64_t)blockIdx.x * nh * nh;
    const int h = 32 * hb + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int g = 32 * gb + 8 * (r >> 2) + 4 * half + (r & 3);
        part_out[g * nh + h] = acc_w[r];
    }
}

// ---------------------------------------------------------------------------
// KV column index remap (PaddleFleet PR #1772, PR body item 2 and description
// part 二): per-batch-local indices of a [b*sq, topk] int32 table become
// flat-global, out = idx >= 0 ? idx + batch * seqlen_kv : pad_value, with
// batch = row / sq.  One pass over the table instead of the unfused route's
// seven elementwise kernels.  Integer work, HBM-bound: 16-byte non-temporal
// vectors when a row is a whole number of vectors.
// ---------------------------------------------------------------------------

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// v + batch*seqlen_kv for v >= 0 (its low 32 bits, as the int64 sum cast to
// int32), else the pad value; `off` = batch*seqlen_kv mod 2^32
__device__ __forceinline__ int32_t remap_one(int32_t v, uint32_t off, int32_t pad) {
    return v >= 0 ? (int32_t)((uint32_t)v + off) : pad;
}

// batch of element (or vector) i, with `per_batch` elements per batch: one
// scalar division per workgroup when a batch spans at least a workgroup
// (then a workgroup holds at most one batch boundary), else per element
template <bool ROWS>
__device__ __forceinline__ int64_t batch_of(int64_t i, int64_t per_batch) {
    const int64_t i0 = linear_block<ROWS>() * blockDim.x;
    if (per_batch >= (int64_t)blockDim.x) {
        const int64_t b0 = i0 / per_batch;
        return b0 + (i >= (b0 + 1) * per_batch ? 1 : 0);
    }
    return i / per_batch;
}

template <bool ROWS>
__global__ __launch_bounds__(256) void kv_remap_vec_kernel(const int32_t* __restrict__ idx,
                                                           int64_t n_vec, int64_t vec_per_batch,
                                                           int64_t seqlen_kv, int32_t pad,
                                                           int32_t* __restrict__ out) {
    const int64_t i = linear_block<ROWS>() * 256 + threadIdx.x;
    if (i >= n_vec) return;
    const uint32_t off = (uint32_t)(batch_of<ROWS>(i, vec_per_batch) * seqlen_kv);
    const i32x4 v = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(idx) + i);
    i32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = remap_one(v[e], off, pad);
    __builtin_nontemporal_store(o, reinterpret_cast<i32x4*>(out) + i);
}

template <bool ROWS>
__global__ __launch_bounds__(256) void kv_remap_scalar_kernel(const int32_t* __restrict__ idx,
                                                              int64_t n, int64_t per_batch,
                                                              int64_t seqlen_kv, int32_t pad,
                                                              int32_t* __restrict__ out) {
    const int64_t i = linear_block<ROWS>() * 256 + threadIdx.x;
    if (i >= n) return;
    out[i] = remap_one(idx[i], (uint32_t)(batch_of<ROWS>(i, per_batch) * seqlen_kv), pad);
}

hipError_t launch_kv_remap(const int32_t* idx, int64_t rows, int64_t sq, int64_t topk,
                           int64_t seqlen_kv, int32_t pad, int32_t* out, hipStream_t stream) {
    const int64_t n = rows * topk;
    if (n == 0) return hipSuccess;
    const bool vec = topk % 4 == 0 && ((uintptr_t)idx & 15u) == 0 && ((uintptr_t)out & 15u) == 0;
    dim3 grid;
    if (vec) {
        const int64_t n_vec = n / 4;
        if (!data_grid((n_vec + 255) / 256, &grid)) return hipErrorInvalidConfiguration;
        auto kern = grid.y > 1 ? kv_remap_vec_kernel<true> : kv_remap_vec_kernel<false>;
        hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, idx, n_vec, (topk / 4) * sq, seqlen_kv, pad, out);
    } else {
        if (!data_grid((n + 255) / 256, &grid)) return hipErrorInvalidConfiguration;
        auto kern = grid.y > 1 ? kv_remap_scalar_kernel<true> : kv_remap_scalar_kernel<false>;
        hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, idx, n, topk * sq, seqlen_kv, pad, out);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// full-width rotary embedding, out of place: out = rope(X) (direction +1) or
// inv_rope(X) (direction -1) on the trailing pe channels of every head row,
// nope channels copied.  The unfused route of PaddleFleet PR #1772 (PR body
// item 1) materialises exactly this tensor before the postmix GEMM, and its
// final backward rebuilds it (rope_full_out_of_place, follow-up commit); it
// is here to run that route on this GPU for comparison.
// Workgroup = (token, group of R head rows), R = min(nh, max(1, 512 / (d/8))).
// Its first R*nope/8 work items copy the nope vectors of the R rows; the last
// R*pe/8 items each produce one pe output vector from its own input vector and
// the partner vector pe/2 channels away.  At d = 512 (R = 8) that is seven
// copy waves and one rotation wave, so no wave mixes the two paths.  Index
// arithmetic is 32-bit apart from the row base.  HBM-bound; 16-byte
// non-temporal loads and stores.
// ---------------------------------------------------------------------------

template <bool ROWS>
__global__ __launch_bounds__(512) void rope_apply_kernel(
    const uint16_t* __restrict__ X, const float* __restrict__ rcos, const float* __restrict__ rsin,
    int64_t table_rows, const int32_t* __restrict__ positions, int64_t sq, int nh, int nope, int pe,
    int rows_per_wg, int groups_per_token, int direction, uint16_t* __restrict__ Out) {
    const int d = nope + pe, h2 = pe >> 1, nv = nope >> 3, pv = pe >> 3;
    int64_t s;  // token
    int h0;     // first head row
    if (!ROWS || blockIdx.y == 0) {  // 32-bit division in the first row
        s = blockIdx.x / (unsigned)groups_per_token;
        h0 = (int)(blockIdx.x - s * groups_per_token) * rows_per_wg;
    } else {
        const int64_t b = linear_block();
        s = b / groups_per_token;
        if (s >= sq) return;
        h0 = (int)(b - s * groups_per_token) * rows_per_wg;
    }
    const int n_copy = rows_per_wg * nv, n_all = rows_per_wg * (nv + pv);
    const float sg = (float)direction;  // +1: turn by +phi, -1: by -phi
    for (int t = threadIdx.x; t < n_all; t += blockDim.x) {
        if (t < n_copy) {
            const int r = t / nv, v = t - r * nv;
            if (h0 + r >= nh) continue;
            const int64_t off = (s * nh + h0 + r) * d + 8 * v;
            const u32x4 val = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(X + off));
            __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(Out + off));
            continue;
        }
        const int u = t - n_copy, r = u / pv, i0 = 8 * (u - r * pv);
        if (h0 + r >= nh) continue;
        const bool first = i0 < h2;
        const int ii = first ? i0 : i0 - h2;
        const int64_t base = (s * nh + h0 + r) * d + nope;
        const u32x4 own = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(X + base + i0));
        const u32x4 par = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(X + base + (first ? i0 + h2 : ii)));
        const int64_t prow = table_row(positions, s, table_rows);
        const f32x4* pc = reinterpret_cast<const f32x4*>(rcos + prow * h2 + ii);
        const f32x4* ps = reinterpret_cast<const f32x4*>(rsin + prow * h2 + ii);
        const f32x4 c0 = pc[0], c1 = pc[1], s0 = ps[0], s1 = ps[1];
        // first half: a C - b S';  second half: b C + a S'  (S' = direction * S)
        const float sp = first ? -sg : sg;
        u32x4 o;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            float r[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int k = 2 * jj + e;
                const float c = k < 4 ? c0[k] : c1[k - 4];
                const float sn = sp * (k < 4 ? s0[k] : s1[k - 4]);
                const float x = bf16_to_f32((own[jj] >> (16 * e)) & 0xffffu);
                const float y = bf16_to_f32((par[jj] >> (16 * e)) & 0xffffu);
                r[e] = x * c + y * sn;
            }
            o[jj] = pack_bf16(r[0], r[1]);
        }
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(Out + base + i0));
    }
}

hipError_t launch_rope_apply(const uint16_t* X, const float* rcos, const float* rsin, int64_t table_rows,
                             const int32_t* positions, int64_t sq, int nh, int nope, int pe, int direction,
                             uint16_t* Out, hipStream_t stream) {
    const int vpr = (nope + pe) / 8;
    if (sq == 0 || vpr == 0) return hipSuccess;
    int rows_per_wg = vpr >= 512 ? 1 : 512 / vpr;
    if (rows_per_wg > nh) rows_per_wg = nh;
    const int groups = (nh + rows_per_wg - 1) / rows_per_wg;
    int threads = (rows_per_wg * vpr + 63) / 64 * 64;
    if (threads > 512) threads = 512;
    dim3 grid;
    if (!data_grid(sq * groups, &grid)) return hipErrorInvalidConfiguration;
    auto kern = grid.y > 1 ? rope_apply_kernel<true> : rope_apply_kernel<false>;
    hipLaunchKernelGGL(kern, grid, dim3(threads), 0, stream, X, rcos, rsin,
                       table_rows, positions, sq, nh, nope, pe, rows_per_wg, groups, direction, Out);
    return hipGetLastError();
}


// ---------------------------------------------------------------------------
// small head counts (nh <= 4): plain fp32 vector arithmetic
//
// With a handful of heads the head mix is a few multiply-adds per element, so
// these kernels use VALU FMAs.  The tiled kernels pack several tokens per
// MFMA tile instead and are faster where they apply (channels in 128- or
// 256-channel parts); these serve the other shapes (d not a multiple of 128,
// or pe wider than a part).
// Workgroup = R consecutive tokens, R = max(1, 512 / (d/8)).  Work items: the
// R*nope/8 nope vectors of the R tokens first, then the R*pe/8 pe vectors, so
// that (at d = 512) whole waves take one path.  A work item is one 8-channel
// vector position of one token, for all heads: it loads the nh input vectors,
// forms out[o] = sum_i M[o][i] in[i] in fp32 (M = W for the forward, W^T for
// dx), and for a pe vector also the partner vector's mix, then turns the pair
// (-phi forward, +phi dx) and rounds once to bf16.
// The weight gradient: the same items accumulate
// sum_c dY[g, c] * inv_rope(O)[h, c] for all (g, h) in fp32 (the rotated
// operand is formed in fp32, no bf16 split); the workgroup adds its items'
// sums in a fixed tree and writes one partial per token block.
// ---------------------------------------------------------------------------

constexpr int SMALL_NH = 4;

__device__ __forceinline__ void bf16x8_to_f32(const u32x4& v, float* f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[2 * j] = __uint_as_float(v[j] << 16);
        f[2 * j + 1] = __uint_as_float(v[j] & 0xffff0000u);
    }
}

template <bool DX, bool ROWS>
__global__ __launch_bounds__(512) void small_mix_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
    const float* __restrict__ rcos, const float* __restrict__ rsin, int64_t table_rows,
    const int32_t* __restrict__ positions, int64_t sq, int nh, int nope, int pe, int tokens_per_wg,
    uint16_t* __restrict__ Out) {
    const int d = nope + pe, h2 = pe >> 1, nv = nope >> 3, pv = pe >> 3;
    float m[SMALL_NH][SMALL_NH];  // m[o][i]
#pragma unroll
    for (int o = 0; o < SMALL_NH; ++o)
#pragma unroll
        for (int i = 0; i < SMALL_NH; ++i)
            m[o][i] = (o < nh && i < nh) ? bf16_to_f32(DX ? W[i * nh + o] : W[o * nh + i]) : 0.0f;
    const int64_t s0 = linear_block<ROWS>() * tokens_per_wg;
    const int n_copy = tokens_per_wg * nv, n_all = tokens_per_wg * (nv + pv);
    for (int t = threadIdx.x; t < n_all; t += blockDim.x) {
        const bool is_pe = t >= n_copy;
        const int u = is_pe ? t - n_copy : t;
        const int per = is_pe ? pv : nv;
        const int r = u / per, v = u - r * per;
        const int64_t s = s0 + r;
        if (s >= sq) continue;
        const int c = is_pe ? nope + 8 * v : 8 * v;
        const uint16_t* xs = X + s * nh * (int64_t)d;
        uint16_t* os = Out + s * nh * (int64_t)d;
        float in[SMALL_NH][8];
#pragma unroll
        for (int i = 0; i < SMALL_NH; ++i) {
            if (i < nh) bf16x8_to_f32(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xs + i * d + c)), in[i]);
        }
        if (!is_pe) {
#pragma unroll
            for (int o = 0; o < SMALL_NH; ++o) {
                if (o >= nh) break;
                float y[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float a = 0.0f;
#pragma unroll
                    for (int i = 0; i < SMALL_NH; ++i)
                        if (i < nh) a += m[o][i] * in[i][e];
                    y[e] = a;
                }
                u32x4 w;
#pragma unroll
                for (int j = 0; j < 4; ++j) w[j] = pack_bf16(y[2 * j], y[2 * j + 1]);
                __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(os + o * d + c));
            }
            continue;
        }
        const int i0 = 8 * v;  // index within the pe channels
        const bool first = i0 < h2;
        const int ii = first ? i0 : i0 - h2;
        const int cp = nope + (first ? i0 + h2 : ii);
        float par[SMALL_NH][8];
#pragma unroll
        for (int i = 0; i < SMALL_NH; ++i) {
            if (i < nh) bf16x8_to_f32(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xs + i * d + cp)), par[i]);
        }
        const int64_t prow = table_row(positions, s, table_rows);
        float cs[8], sn[8];
        {
            const f32x4 c0 = *reinterpret_cast<const f32x4*>(rcos + prow * h2 + ii);
            const f32x4 c1 = *reinterpret_cast<const f32x4*>(rcos + prow * h2 + ii + 4);
            const f32x4 q0 = *reinterpret_cast<const f32x4*>(rsin + prow * h2 + ii);
            const f32x4 q1 = *reinterpret_cast<const f32x4*>(rsin + prow * h2 + ii + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) { cs[e] = c0[e]; cs[4 + e] = c1[e]; sn[e] = q0[e]; sn[4 + e] = q1[e]; }
        }
        // forward (-phi): first half a C + b S, second half a C - b S;  dx (+phi): the signs swapped
        const float sg = (first != DX) ? 1.0f : -1.0f;
#pragma unroll
        for (int o = 0; o < SMALL_NH; ++o) {
            if (o >= nh) break;
            float y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float a = 0.0f, b = 0.0f;
#pragma unroll
                for (int i = 0; i < SMALL_NH; ++i)
                    if (i < nh) { a += m[o][i] * in[i][e]; b += m[o][i] * par[i][e]; }
                y[e] = a * cs[e] + sg * (b * sn[e]);
            }
            u32x4 w;
#pragma unroll
            for (int j = 0; j < 4; ++j) w[j] = pack_bf16(y[2 * j], y[2 * j + 1]);
            __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(os + o * d + c));
        }
    }
}

// one weight-gradient partial per block of tokens (block b of B = gridDim.x:
// tokens [b*sq/B, (b+1)*sq/B)); 256 threads
__global__ __launch_bounds__(256) void small_dw_kernel(
    const uint16_t* __restrict__ dY, const uint16_t* __restrict__ O,
    const float* __restrict__ rcos, const float* __restrict__ rsin, int64_t table_rows,
    const int32_t* __restrict__ positions, int64_t sq, int nh, int nope, int pe,
    float* __restrict__ partials, int spans) {
    constexpr int NN = SMALL_NH * SMALL_NH;
    __shared__ float red[NN][256];
    const int d = nope + pe, h2 = pe >> 1, nv = nope >> 3, pv = pe >> 3;
    // token block tb of B = gridDim.x / spans, vector span y of each token's
    // d/8 vectors (spans > 1 only for very wide rows)
    const int64_t nbt = gridDim.x / spans, tb = blockIdx.x / spans;
    const int y = (int)(blockIdx.x - tb * spans);
    const int64_t s0 = tb * sq / nbt;
    const int64_t s1 = (tb + 1) * sq / nbt;
    const int v_all = nv + pv;
    const int v0 = (int)((int64_t)y * v_all / spans);
    const int vpr = (int)((int64_t)(y + 1) * v_all / spans) - v0;
    const int64_t n_items = (s1 - s0) * vpr;
    float acc[NN];
#pragma unroll
    for (int k = 0; k < NN; ++k) acc[k] = 0.0f;
    for (int64_t it = threadIdx.x; it < n_items; it += 256) {
        const int64_t r = it / vpr;
        const int v = v0 + (int)(it - r * vpr);
        const int64_t s = s0 + r;
        const bool is_pe = v >= nv;
        const int c = 8 * v;  // nope vectors first, then pe vectors, in channel order
        const uint16_t* ys = dY + s * nh * (int64_t)d;
        const uint16_t* os = O + s * nh * (int64_t)d;
        float g[SMALL_NH][8], x[SMALL_NH][8];
#pragma unroll
        for (int i = 0; i < SMALL_NH; ++i) {
            if (i < nh) {
                bf16x8_to_f32(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ys + i * d + c)), g[i]);
                bf16x8_to_f32(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(os + i * d + c)), x[i]);
            }
        }
        if (is_pe) {  // x <- inv_rope(O) for these 8 channels, in fp32
            const int i0 = c - nope;
            const bool first = i0 < h2;
            const int ii = first ? i0 : i0 - h2;
            const int cp = nope + (first ? i0 + h2 : ii);
            const int64_t prow = table_row(positions, s, table_rows);
            float cs[8], sn[8];
            const f32x4 c0 = *reinterpret_cast<const f32x4*>(rcos + prow * h2 + ii);
            const f32x4 c1 = *reinterpret_cast<const f32x4*>(rcos + prow * h2 + ii + 4);
            const f32x4 q0 = *reinterpret_cast<const f32x4*>(rsin + prow * h2 + ii);
            const f32x4 q1 = *reinterpret_cast<const f32x4*>(rsin + prow * h2 + ii + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) { cs[e] = c0[e]; cs[4 + e] = c1[e]; sn[e] = q0[e]; sn[4 + e] = q1[e]; }
            const float sg = first ? 1.0f : -1.0f;  // -phi: first half a C + b S, second a C - b S
#pragma unroll
            for (int i = 0; i < SMALL_NH; ++i) {
                if (i >= nh) break;
                float p[8];
                bf16x8_to_f32(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(os + i * d + cp)), p);
#pragma unroll
                for (int e = 0; e < 8; ++e) x[i][e] = x[i][e] * cs[e] + sg * (p[e] * sn[e]);
            }
        }
#pragma unroll
        for (int a = 0; a < SMALL_NH; ++a)
#pragma unroll
            for (int b = 0; b < SMALL_NH; ++b) {
                if (a >= nh || b >= nh) continue;
                float t = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) t += g[a][e] * x[b][e];
                acc[a * SMALL_NH + b] += t;
            }
    }
    // fixed-order tree over the 256 threads
#pragma unroll
    for (int k = 0; k < NN; ++k) red[k][threadIdx.x] = acc[k];
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) {
#pragma unroll
            for (int k = 0; k < NN; ++k) red[k][threadIdx.x] += red[k][threadIdx.x + w];
        }
        __syncthreads();
    }
    if ((int)threadIdx.x < nh * nh) {
        const int a = threadIdx.x / nh, b = threadIdx.x % nh;
        partials[(int64_t)blockIdx.x * nh * nh + threadIdx.x] = red[a * SMALL_NH + b][0];
    }
}

// ---------------------------------------------------------------------------
// host-side launchers (argument checks are done by the caller)
// ---------------------------------------------------------------------------

static constexpr size_t kMaxLds = 160 * 1024;  // LDS per workgroup on gfx950

// A kernel attribute set once per device: hipFuncSetAttribute acts on the
// current device, so bit d records device d (devices from 64 on set it on
// every launch).  Idempotent: a race only repeats the call.
struct AttrPerDevice {
    std::atomic<uint64_t> done{0};
    template <class Set>
    hipError_t ensure(Set&& set) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t)1 << dev : 0;
        if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
        e = set();
        if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
        return e;
    }
};

template <int NHP, int MPI, bool DX>
static hipError_t launch_mix_t(const MixArgs& a, hipStream_t stream) {
    const int d = a.nope + a.pe;
    (void)d;
    const int nu = (a.nope + 15) / 16 + (a.pe / 2) / 8;
    const int mbt = (nu + 1) / 2;
    const int ipt = (mbt + MPI - 1) / MPI;
    const int64_t total = a.sq * ipt;
    int64_t grid = (int64_t)a.n_cu * a.waves_per_cu;
    if (grid > total) grid = total;
    if (grid < 1) return hipSuccess;
    hipLaunchKernelGGL((mix_kernel<NHP, MPI, DX>), dim3((unsigned)grid), dim3(64), 0, stream, a.X,
                       a.W, a.rcos, a.rsin, a.table_rows, a.positions, a.nh, a.nope, a.pe, a.Out,
                       total, ipt);
    return hipGetLastError();
}

// token-part kernel: one workgroup per tile = (token, CP-channel part)
template <int NH, int CP, int WAVES, bool DX, int NS = 1>
static hipError_t launch_part_t(const MixArgs& a, hipStream_t stream) {
    using C = PartCfg<NH, CP, WAVES, NS>;
    using CP_ = PartCfg<NH, CP, WAVES, NS, true>;  // padded tiles (their own row pitch)
    const int d = a.nope + a.pe;
    const int cpt = d / CP;
    const bool pad = a.nh != NH;
    const int tp = pad ? C::tokens_per_tile(a.nh, a.pe) : 1;
    const int64_t n_tiles = (a.sq + tp - 1) / tp * cpt;
    const size_t lds = pad ? CP_::lds_bytes(a.nope, a.pe, tp) : C::lds_bytes(a.nope, a.pe, tp);
    auto kern = pad ? mix_part_kernel<NH, CP, WAVES, DX, NS, true> : mix_part_kernel<NH, CP, WAVES, DX, NS, false>;
    static AttrPerDevice attr[2];
    const hipError_t ae = attr[pad].ensure([&] {
        // largest: pe = CP with the scratch
        size_t lds_max = (pad ? CP_::lds_bytes(8, CP) : C::lds_bytes(8, CP)) + (size_t)C::NT * 16;
        if (lds_max > kMaxLds) lds_max = kMaxLds;  // shapes beyond it are not routed here
        if (lds_max <= 65536) return hipSuccess;
        return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_max);
    });
    if (ae != hipSuccess) return ae;
    dim3 grid;
    if (!data_grid(n_tiles, &grid)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(kern, grid, dim3(64 * WAVES), lds, stream, a.X, a.W, a.rcos,
                       a.rsin, a.table_rows, a.positions, a.sq, a.nh, a.nope, a.pe, cpt, tp, n_tiles, a.Out);
    return hipGetLastError();
}

// Head rows of the token-part tile for nh heads: 32, 64 or 128 (padded with zeros).
int mix_padded_heads(int nh) { return nh <= 32 ? 32 : (nh <= 64 ? 64 : 128); }

// Tokens per 64-row tile of the token-part kernel with CP-channel parts.
static int mix_tokens_per_tile64(int nh, int pe, int cp) {
    return cp == 256 ? PartCfg<64, 256, 8>::tokens_per_tile(nh, pe) : PartCfg<64, 128, 4>::tokens_per_tile(nh, pe);
}

// Head rows of the forward/dx tile: 64 for nh <= 64 (several tokens per tile
// when nh <= 32), 96 (three 32-head N-blocks, split over 3 wave groups of 2
// waves) or 128.  The forward also takes 32-row tiles where they measured
// faster: nh = 32 (exact rows, 16-byte W loads), and where the angle rows
// would leave a 64-row tile half empty anyway (nh = 1).  dx keeps 64 rows:
// the fused backward computes dO in the same tiles (same tokens per tile,
// same MFMA inputs and order), so the two agree bit for bit.
static int mix_tile_heads(int nh, int pe, int cp, bool dx) {
    if (nh > 64) return nh <= 96 ? 96 : 128;
    if (dx) return 64;
    if (nh == 32) return 32;
    return mix_tokens_per_tile64(nh, pe, cp) * nh <= 32 ? 32 : 64;
}

// Channel-part width of the token-part kernel for this shape, or 0 when the
// shape needs another kernel: 4 < nh <= 128 (padded to 32, 64 or 128), the part must
// divide d, hold the whole pe range, fit the workgroup's LDS, and the grid
// must stay below 2^31.
int mix_part_width(int64_t sq, int nh, int nope, int pe) {
    if (nh < 1 || nh > 128) return 0;
    const int nhp = mix_padded_heads(nh);
    const int d = nope + pe;
    const int cands[2] = {256, 128};
    for (int cp : cands) {
        if (d % cp != 0 || pe > cp) continue;
        if (nhp == 128 && cp == 256 && PartCfg<128, 256, 8, 4>::lds_bytes(nope, pe) > kMaxLds) continue;
        if (sq * (int64_t)(d / cp) >= ((int64_t)1 << 31)) return 0;
        return cp;
    }
    return 0;
}

template <bool DX>
static hipError_t launch_mix_dx(const MixArgs& a, hipStream_t stream) {
    const bool w16 = ((uintptr_t)a.W & 15u) == 0;
    // the tiled kernels read W with 16-byte loads when nh fills the padded rows exactly
    int cp = a.force_general ? 0 : mix_part_width(a.sq, a.nh, a.nope, a.pe);
    const int nhp = cp ? mix_tile_heads(a.nh, a.pe, cp, DX) : 0;
    if (!w16 && a.nh == nhp) cp = 0;
    if (cp == 256 && nhp == 64) return launch_part_t<64, 256, 8, DX>(a, stream);
    if (cp == 128 && nhp == 64) return launch_part_t<64, 128, 4, DX>(a, stream);
    if (cp == 256 && nhp == 32) return launch_part_t<32, 256, 8, DX>(a, stream);
    if (cp == 128 && nhp == 32) return launch_part_t<32, 128, 4, DX>(a, stream);
    if (cp == 256 && nhp == 96) return launch_part_t<96, 256, 6, DX, 3>(a, stream);   // N split in 3
    if (cp == 128 && nhp == 96) return launch_part_t<96, 128, 6, DX, 3>(a, stream);
    if (cp == 256 && nhp == 128) return launch_part_t<128, 256, 8, DX, 4>(a, stream);  // N split in 4
    if (cp == 128 && nhp == 128) return launch_part_t<128, 128, 8, DX, 4>(a, stream);
    if (!a.force_general && a.nh <= SMALL_NH) {
        const int vpr = (a.nope + a.pe) / 8;
        const int tok = vpr >= 512 ? 1 : 512 / vpr;
        int threads = (tok * vpr + 63) / 64 * 64;
        if (threads > 512) threads = 512;
        dim3 grid;
        if (!data_grid((a.sq + tok - 1) / tok, &grid)) return hipErrorInvalidConfiguration;
        auto kern = grid.y > 1 ? small_mix_kernel<DX, true> : small_mix_kernel<DX, false>;
        hipLaunchKernelGGL(kern, grid, dim3(threads), 0, stream, a.X, a.W,
                           a.rcos, a.rsin, a.table_rows, a.positions, a.sq, a.nh, a.nope, a.pe, tok, a.Out);
        return hipGetLastError();
    }
    if (a.nh <= 16) return launch_mix_t<16, 2, DX>(a, stream);
    if (a.nh <= 32) return launch_mix_t<32, 2, DX>(a, stream);
    if (a.nh <= 64) return launch_mix_t<64, 2, DX>(a, stream);
    return launch_mix_t<128, 1, DX>(a, stream);
}

hipError_t launch_mix(const MixArgs& a, bool dx, hipStream_t stream) {
    return dx ? launch_mix_dx<true>(a, stream) : launch_mix_dx<false>(a, stream);
}

// Tokens per weight-gradient block: sq*max(nh, 64)/32768 rounded up to a
// multiple of 4 (at least 4).  At sq=16384, nh=64 that is 32 tokens, 512
// blocks: two resident workgroups on each of 256 CUs, one round.  Below 64
// heads the chunks hold several tokens, so the block count stays at 512 for
// the same number of chunks per block.
int dw_tokens_per_block(int64_t sq, int nh) {
    int64_t t = (sq * (nh < 64 ? 64 : nh) + 32767) / 32768;
    t = (t + 3) / 4 * 4;
    if (t < 4) t = 4;
    if (t > (1 << 20)) t = 1 << 20;
    return (int)t;
}

// Blocks of the weight-gradient kernels: the count that blocks of
// dw_tokens_per_block tokens give, unless that leaves the last round of
// resident workgroups (two per CU up to 64 head rows, one at 128, on
// gfx950's 256 CUs) less than three quarters full; then it is rounded to the
// nearest multiple of a round.  The tokens are spread evenly over the blocks
// (block b holds tokens [b*sq/B, (b+1)*sq/B)).  Constants, not the device's
// CU count: the partition, and with it the summation order, depends on the
// shape only.
int64_t dw_num_blocks(int64_t sq, int nh) {
    const int t = dw_tokens_per_block(sq, nh);
    const int64_t round = nh > 64 ? 256 : 512;
    int64_t b = (sq + t - 1) / t;
    if (b > round && b % round < round * 3 / 4) {
        b = (b + round / 2) / round * round;
        if (b > sq) b = sq;
    }
    return b;
}

// Each weight-gradient partial accumulates its products in fp32 chains, one
// add per MFMA k-step (16 channels of one token); the error of such a chain
// grows with its length (like 2^-24 * sqrt(length) for random data: one
// token of 2^24 channels at 128 heads, a chain of 2^20, measured 1.05e-4
// relative).  No chain is allowed more than kMaxChain k-steps.  A token (or a
// group of tokens sharing a chunk) adds at most ceil(d/16) k-steps to a
// chain; blocks whose units would exceed the cap are made smaller, and a
// single unit that exceeds it is split into channel spans, each with its own
// partial.  Shapes within the cap (every shape of fewer than 2^14 channels
// per unit-block product, e.g. the production blocks of 16 or 32 tokens of
// 512 channels: 512 or 1024 k-steps) keep the plain partition and its bits.
static constexpr int64_t kMaxChain = (int64_t)1 << 14;

static DwPlan chain_capped(int64_t units, int64_t nb0, int d) {
    DwPlan p{nb0, 1};
    if (units <= 0 || nb0 <= 0) return p;
    const int64_t per_unit = ((int64_t)d + 15) / 16;
    if ((units + nb0 - 1) / nb0 * per_unit <= kMaxChain) return p;
    if (per_unit <= kMaxChain) {
        const int64_t u = kMaxChain / per_unit;  // units per block; even spreading keeps <= u
        p.blocks = (units + u - 1) / u;
        return p;
    }
    p.blocks = units;
    p.spans = (int)((per_unit + kMaxChain - 1) / kMaxChain);  // <= d/128: whole 128-channel parts
    return p;
}

DwPlan dw_plan(int64_t sq, int nh, int nope, int pe) {
    return chain_capped(sq, dw_num_blocks(sq, nh), nope + pe);
}

// chunk width of the fused backward: 256 channels (16 waves) where d allows
static int bwd_fused_chunk(int d) { return d % 256 == 0 ? 256 : 128; }

// Head rows of the fused backward's chunks: 64 (several tokens per chunk
// below 33 heads, padded rows above), 96 for 64 < nh <= 96 where d is a
// multiple of 256 and the 256-channel chunks fit the LDS (pe rotated in
// registers or absent), else 128 (128-channel chunks; their rows are 256 B
// segments, which stream slower than the 512 B of 256-channel chunks).
static bool bwd_fused96_fits(int nope, int pe);
static int bwd_fused_rows(int nh, int nope, int pe) {
    if (nh <= 64) return 64;
    if (nh <= 96 && (nope + pe) % 256 == 0 && bwd_fused96_fits(nope, pe)) return 96;
    return 128;
}

// Tokens per chunk of the fused backward: nh <= 32 packs the tokens of the
// dx tile (the token-part kernel's 64-row tile with parts as wide as the
// chunks), so the two compute dO identically; otherwise one.
static int bwd_fused_tokens_per_chunk(int nh, int nope, int pe) {
    return nh <= 32 ? mix_tokens_per_tile64(nh, pe, bwd_fused_chunk(nope + pe)) : 1;
}

// The fused backward aims at blocks of half as many tokens as the weight
// gradient: sq*max(nh, 64)/65536 rounded up to a multiple of 4 (at least 4),
// then to a multiple of the tokens per chunk (whole chunks, aligned with the
// dx tiles).  Its one 16-wave workgroup per CU then works through four rounds
// of blocks at the production shape, which balances better than two.
int bwd_fused_tokens_per_block(int64_t sq, int nh, int nope, int pe) {
    int64_t t = (sq * (nh < 64 ? 64 : nh) + 65535) / 65536;
    t = (t + 3) / 4 * 4;
    if (t < 4) t = 4;
    if (t > (1 << 20)) t = 1 << 20;
    const int tp = bwd_fused_tokens_per_chunk(nh, nope, pe);
    t = (t + tp - 1) / tp * tp;
    return (int)t;
}

// Blocks of the fused backward.  The count that blocks of
// bwd_fused_tokens_per_block tokens give is kept unless it leaves the last
// round of kFusedRound blocks (one workgroup on each of gfx950's 256 CUs)
// less than three quarters full; then it is rounded to the nearest multiple
// of kFusedRound and the token groups are spread evenly over the blocks
// (nh = 96 at 1 GiB: 547 -> 512 blocks, 1000 -> 776 us).  With blocks of one
// group the nearest multiple can exceed the groups: below two rounds the
// count is then one round (nh = 3 at sq = 8192: 391 -> 256 blocks of one or
// two groups, 30.6 -> 27.6 us), else one block per group (nh = 5: 683 ->
// 512 blocks measured 43.6 -> 47.5 us).  A constant, not
// the device's CU count: the partition, and with it the weight gradient's
// summation order, depends on the shape only.
static constexpr int64_t kFusedRound = 256;
static int64_t bwd_fused_num_blocks(int64_t sq, int nh, int nope, int pe) {
    const int t = bwd_fused_tokens_per_block(sq, nh, nope, pe);
    const int tp = bwd_fused_tokens_per_chunk(nh, nope, pe);
    const int64_t groups = (sq + tp - 1) / tp, per_block = t / tp;
    int64_t b = (groups + per_block - 1) / per_block;
    if (b > kFusedRound && b % kFusedRound < kFusedRound * 3 / 4) {
        b = (b + kFusedRound / 2) / kFusedRound * kFusedRound;
        // more blocks than token groups: with fewer than two rounds of
        // groups, one round of blocks of one or two groups; otherwise one
        // group per block
        if (b > groups) b = groups < 2 * kFusedRound ? kFusedRound : groups;
    }
    return b;
}

// The fused backward's plan: units are token groups (one chunk's tokens).
DwPlan bwd_fused_plan(int64_t sq, int nh, int nope, int pe) {
    const int tp = bwd_fused_tokens_per_chunk(nh, nope, pe);
    return chain_capped((sq + tp - 1) / tp, bwd_fused_num_blocks(sq, nh, nope, pe), nope + pe);
}

// Chunk width of the LDS-staged weight-gradient kernel, or 0 for the direct kernel.
int dw_chunk_width(int nh, int nope, int pe) {
    if (nh < 1 || nh > 128) return 0;  // padded to 32, 64 or 128 rows
    const int d = nope + pe;
    return (d % 128 == 0 && pe <= 128) ? 128 : 0;
}

// Tokens per chunk of the weight-gradient kernel with NH head rows: as many
// as fill the rows, while each quad of every token's cos and sin rows has a
// thread to load it.
template <int NH>
static int dw_tokens_per_chunk(int nh, int pe) {
    if (nh >= NH) return 1;
    int tp = NH / nh;
    const int cap = pe > 0 ? 8 * DwCfg<NH, 128>::NT / pe : tp;
    return tp < cap ? tp : (cap < 1 ? 1 : cap);
}

// Head rows of the weight-gradient chunk: 64 (several tokens per chunk when
// nh <= 32), 32 when the angle rows would leave a 64-row chunk half empty
// anyway, 128 for nh > 64.
static int dw_tile_heads(int nh, int pe) {
    if (nh > 64) return 128;
    return dw_tokens_per_chunk<64>(nh, pe) * nh <= 32 ? 32 : 64;
}

template <int NHC>
static hipError_t launch_dw_chunk_t(const DwArgs& a, const DwPlan& pl, hipStream_t stream) {
    const bool pad = a.nh != NHC;
    const int tp = pad ? dw_tokens_per_chunk<NHC>(a.nh, a.pe) : 1;
    auto kern = pad ? dw_chunk_kernel<NHC, 128, true> : dw_chunk_kernel<NHC, 128, false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)pl.partials()), dim3(DwCfg<NHC, 128>::NT), 0, stream, a.dY, a.O,
                       a.rcos, a.rsin, a.table_rows, a.positions, a.sq, a.nh, a.nope, a.pe, a.partials, tp,
                       pl.spans);
    return hipGetLastError();
}

template <int NHP>
static hipError_t launch_dw_t(const DwArgs& a, hipStream_t stream) {
    const DwPlan pl = dw_plan(a.sq, a.nh, a.nope, a.pe);
    if (pl.partials() > INT32_MAX) return hipErrorInvalidValue;
    const int ch = a.force_general ? 0 : dw_chunk_width(a.nh, a.nope, a.pe);
    if (ch == 128) {
        const int nhc = dw_tile_heads(a.nh, a.pe);
        const hipError_t e = nhc == 32   ? launch_dw_chunk_t<32>(a, pl, stream)
                             : nhc == 64 ? launch_dw_chunk_t<64>(a, pl, stream)
                                         : launch_dw_chunk_t<128>(a, pl, stream);
        if (e != hipSuccess) return e;
    } else if (!a.force_general && a.nh <= SMALL_NH) {
        hipLaunchKernelGGL(small_dw_kernel, dim3((unsigned)pl.partials()), dim3(256), 0, stream, a.dY, a.O,
                           a.rcos, a.rsin, a.table_rows, a.positions, a.sq, a.nh, a.nope, a.pe, a.partials,
                           pl.spans);
    } else {
        hipLaunchKernelGGL((dw_partial_kernel<NHP>), dim3((unsigned)pl.partials()), dim3(256), 0, stream,
                           a.dY, a.O, a.rcos, a.rsin, a.table_rows, a.positions, a.sq, a.nh, a.nope, a.pe,
                           a.partials, pl.spans);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t ne = (int64_t)a.nh * a.nh;
    hipLaunchKernelGGL(dw_reduce_kernel, dim3((unsigned)((ne + 63) / 64)), dim3(1024), 0, stream,
                       a.partials, pl.partials(), ne, a.dW);
    return hipGetLastError();
}

static bool bwd_fused96_fits(int nope, int pe) {
    return (pe == 0 || pe_pairs_in_blocks(nope, pe)) &&
           BwdCfg<96, 256, 12>::lds_bytes(nope, pe, BwdCfg<96, 256, 12>::rope_group(1), false) <= kMaxLds;
}

// fused backward (dx + dW partials in one pass), then the fixed-order reduce
bool bwd_fused_applies(int nh, int nope, int pe) {
    const int d = nope + pe;
    if (nh < 1 || d % 128 != 0 || pe > 128 || d > (1 << 24)) return false;
    // several tokens per 64-row chunk (nh <= 32; at most a cos/sin group of them),
    // head rows padded to 64 (32 < nh <= 64), or to 128 (pe rotated in registers only);
    // the LDS (chunk buffers, W or the pe scratch, two cos/sin groups) must fit
    size_t lds;
    if (nh <= 64) {
        const int tp = bwd_fused_tokens_per_chunk(nh, nope, pe);
        if (tp > BwdCfg<64, 128, 8>::RG_MAX) return false;
        const int rgt = BwdCfg<64, 128, 8>::rope_group(tp);
        lds = bwd_fused_chunk(d) == 256 ? BwdCfg<64, 256, 16>::lds_bytes(nope, pe, rgt, false)
                                        : BwdCfg<64, 128, 8>::lds_bytes(nope, pe, rgt, false);
    } else {
        if (!(pe == 0 || pe_pairs_in_blocks(nope, pe))) return false;
        if (bwd_fused_rows(nh, nope, pe) == 96) return true;
        lds = BwdCfg<128, 128, 16>::lds_bytes(nope, pe, BwdCfg<128, 128, 16>::rope_group(1), false);
    }
    return lds <= kMaxLds;
}

template <int NH, int CH, int WAVES>
static hipError_t launch_bwd_fused_t(const MixArgs& mx, const DwArgs& a, int64_t ngroups, const DwPlan& pl,
                                     int tp, hipStream_t stream) {
    using C = BwdCfg<NH, CH, WAVES>;
    const bool pad = a.nh != NH;
    const int rgt = C::rope_group(tp);
    // The pe operand formed once per chunk (where its lo area fits the LDS):
    // at NH = 128 four waves per row block each rotated it in four k-steps
    // per chunk (rotation 70 us of 721 us at sq = 8192), and this takes the
    // backward from 732 to 712 us.  At NH = 64 its registers pushed spill
    // reloads into the chunk loop (535 -> 730 us), so it is not compiled there.
    // 128 rows only: with 64 rows the dW waves rotating their own pe operand
    // measured faster (the extra staging-phase barrier costs more there)
    constexpr bool PS_OK = NH == 128;
    const int vh = a.pe / 8;  // its tasks per row: a power of two
    const bool ps = PS_OK && a.pe > 0 && (vh & (vh - 1)) == 0 && C::lds_bytes(a.nope, a.pe, rgt, true) <= kMaxLds;
    // Direct dO stores (waves split by gradient): the dx waves' dO rows are a
    // plain copy (pe rotated in registers or absent) and every paired pe
    // block's partner columns lie in the same wave's channels.  Against the
    // store phase, in the benchmark's regime (settled): 64 rows 549-552 ->
    // 533-534 us (510 -> 516), 96 rows at nh = 96, sq = 8192 522-528 ->
    // 518-521 us (477 -> 456), 128 rows at nh = 128, sq = 8192 651-654 ->
    // 619-624 us (593 -> 582).
    constexpr bool DST_OK = C::SPLIT;
    constexpr int DXW = C::NB == 2 ? 2 : C::DXM;  // M-blocks per dx wave with direct stores
    const int L32 = (a.nope % CH) / 32;            // first pe M-block of its chunk
    const bool dst = DST_OK && (a.pe == 0 || (pe_pairs_in_blocks(a.nope, a.pe) &&
                                              L32 / DXW == (L32 + a.pe / 32 - 1) / DXW));
    auto kern = pad ? (ps ? (dst ? bwd_fused_kernel<NH, CH, WAVES, true, PS_OK, DST_OK>
                                 : bwd_fused_kernel<NH, CH, WAVES, true, PS_OK, false>)
                          : (dst ? bwd_fused_kernel<NH, CH, WAVES, true, false, DST_OK>
                                 : bwd_fused_kernel<NH, CH, WAVES, true, false, false>))
                    : (ps ? (dst ? bwd_fused_kernel<NH, CH, WAVES, false, PS_OK, DST_OK>
                                 : bwd_fused_kernel<NH, CH, WAVES, false, PS_OK, false>)
                          : (dst ? bwd_fused_kernel<NH, CH, WAVES, false, false, DST_OK>
                                 : bwd_fused_kernel<NH, CH, WAVES, false, false, false>));
    static AttrPerDevice attr[2][2][2];
    const hipError_t ae = attr[pad][ps][dst].ensure([&] {
        size_t lds_max = C::lds_bytes(8, 128, C::RG_MAX, true);  // largest: pe = 128 with the scratch
        if (lds_max > kMaxLds) lds_max = kMaxLds;
        return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_max);
    });
    if (ae != hipSuccess) return ae;
    const size_t lds = C::lds_bytes(a.nope, a.pe, rgt, ps);
    if (lds > kMaxLds) return hipErrorInvalidValue;  // excluded by bwd_fused_applies
    hipLaunchKernelGGL(kern, dim3((unsigned)pl.partials()), dim3(C::NT), lds, stream, a.dY, a.O, mx.W, a.rcos,
                       a.rsin, a.table_rows, a.positions, a.sq, a.nh, a.nope, a.pe, mx.Out, a.partials, ngroups, tp,
                       rgt, pl.spans);
    return hipGetLastError();
}

hipError_t launch_bwd_fused(const MixArgs& mx, const DwArgs& a, hipStream_t stream) {
    const DwPlan pl = bwd_fused_plan(a.sq, a.nh, a.nope, a.pe);
    if (pl.partials() > INT32_MAX) return hipErrorInvalidValue;
    const int tp = bwd_fused_tokens_per_chunk(a.nh, a.nope, a.pe);
    const int64_t ngroups = (a.sq + tp - 1) / tp;
    hipError_t err;
    if (a.nh > 64)
        err = bwd_fused_rows(a.nh, a.nope, a.pe) == 96 ? launch_bwd_fused_t<96, 256, 12>(mx, a, ngroups, pl, 1, stream)
                                                       : launch_bwd_fused_t<128, 128, 16>(mx, a, ngroups, pl, 1, stream);
    else
        err = bwd_fused_chunk(a.nope + a.pe) == 256 ? launch_bwd_fused_t<64, 256, 16>(mx, a, ngroups, pl, tp, stream)
                                                    : launch_bwd_fused_t<64, 128, 8>(mx, a, ngroups, pl, tp, stream);
    if (err != hipSuccess) return err;
    const int64_t ne = (int64_t)a.nh * a.nh;
    hipLaunchKernelGGL(dw_reduce_kernel, dim3((unsigned)((ne + 63) / 64)), dim3(1024), 0, stream,
                       a.partials, pl.partials(), ne, a.dW);
    return hipGetLastError();
}

hipError_t launch_dw(const DwArgs& a, hipStream_t stream) {
    if (a.nh <= 16) return launch_dw_t<16>(a, stream);
    if (a.nh <= 32) return launch_dw_t<32>(a, stream);
    if (a.nh <= 64) return launch_dw_t<64>(a, stream);
    return launch_dw_t<128>(a, stream);
}

hipError_t launch_rope_table(double theta, int pe, int64_t rows, float* cos_out, float* sin_out,
                             int n_cu, hipStream_t stream) {
    const int64_t n = rows * (pe / 2);
    if (n == 0) return hipSuccess;
    int64_t grid = (n + 255) / 256;
    const int64_t cap = (int64_t)n_cu * 32;
    if (grid > cap) grid = cap;
    hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)grid), dim3(256), 0, stream, theta, pe,
                       rows, cos_out, sin_out);
    return hipGetLastError();
}

}  // namespace pm
