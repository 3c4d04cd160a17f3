// asf_kernels.hip -- gfx950 kernels of the activation-sparse FFN decode path.
//
// Steps of one decode step of one layer:
//   pred_l1   h = ReLU(P1 x + c1)                  dense GEMV, one wave per row
//   pred_l2   s = P2 h + c2, bit = s > theta      dense GEMV over slot-ordered rows;
//             64 rows -> one uint64 mask word      8 rows per wave, 8 waves per word
//   compact   union of the tokens' masks, popcount + prefix sum -> ascending
//             slot list (and original ids through the neuron table)
//   ffn       per active neuron: FC1 dot of its up row with x (+b1, ReLU; or the
//             ReLU-gated form), then AXPY of its down column into y; each
//             workgroup owns a float32 partial of y
//   reduce    y = residual + b2 + sum of the partials, in a fixed order
//
// The steps exist as separate kernels (asf_predict, asf_sparse_ffn) and fused
// into one cooperative kernel per decode step (k_decode) that separates them
// with grid barriers and issues the loads of its predictor layer-2 rows before
// the first barrier, so the whole predictor streams from HBM at once.  Both
// forms share the per-row, per-neuron and per-tile device code below, so they
// produce the same bits.
//
// All weight reads are whole 16-byte chunks (64 lanes x 16 B = 1 KiB per wave
// instruction) of contiguous rows: an active neuron's up row and down column
// sit back to back in one bundle, so its bytes form one contiguous run
// ("LLM模型之PowerInfer1.0", "其他" question 3: load the active columns of the
// down projection contiguously and skip the inactive ones).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "asf_internal.h"

namespace asf {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kWaves = kFfnThreads / 64;       // waves per 512-thread workgroup
constexpr int kL2Rows = 8;                     // predictor layer-2 rows per wave
constexpr uint64_t kSpinTicks = 100000000ull;  // 1 s of the 100 MHz realtime clock

// elements per 16-byte chunk: 8 binary16 or 4 binary32
template <int WT> struct Elt { static constexpr int E = WT ? 8 : 4; };

template <int WT>
__device__ __forceinline__ void unpack(const u32x4 c, float *v) {
    if constexpr (WT == 1) {
        f16x8 h = __builtin_bit_cast(f16x8, c);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (float)h[e];
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(c[e]);
    }
}

template <int E>
__device__ __forceinline__ void load_f32(const float *p, float *v) {
    const float4 *q = reinterpret_cast<const float4 *>(p);
#pragma unroll
    for (int k = 0; k < E / 4; ++k) {
        float4 t = q[k];
        v[4 * k + 0] = t.x;
        v[4 * k + 1] = t.y;
        v[4 * k + 2] = t.z;
        v[4 * k + 3] = t.w;
    }
}

// Butterfly sum over the 64 lanes of a wave.  Each step adds a pair in both
// lanes of the pair, so every lane ends with the same bits.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// ---------------------------------------------------------------- grid barrier
// Sense-reversing barrier over the workgroups of a cooperative launch (all
// co-resident).  bar[0] counts arrivals, bar[1] is the generation.  Each wave
// first waits for its own stores; thread 0 then arrives with an acquire-
// release RMW (one L2 write-back per workgroup), the last arrival resets the
// count and bumps the generation (release), and the others poll the
// generation with relaxed loads and take one acquire fence when it moves.
// Waits are bounded: after about a second without progress the error word
// gets bit 0 and the wait ends, so a fault in the protocol cannot hang the
// device.
__device__ void grid_sync(unsigned *bar, unsigned nblocks, int *err) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned gen = __hip_atomic_load(bar + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const unsigned arrived =
            __hip_atomic_fetch_add(bar, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (arrived + 1u == nblocks) {
            __hip_atomic_store(bar, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_add(bar + 1, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            const uint64_t t0 = wall_clock64();
            while (__hip_atomic_load(bar + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gen) {
                __builtin_amdgcn_s_sleep(1);
                if (wall_clock64() - t0 > kSpinTicks) {
                    atomicOr(err, 1);
                    break;
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
    }
    __syncthreads();
}

// ---------------------------------------------------------------- layout
__global__ void k_perm_rows(const u32x4 *__restrict__ src, int C, const int32_t *__restrict__ perm,
                            int nrows, u32x4 *__restrict__ dst, size_t dstride, size_t doff) {
    const size_t total = (size_t)nrows * C;
    for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (size_t)gridDim.x * blockDim.x) {
        const int r = (int)(idx / C), c = (int)(idx % C);
        int sr = perm ? perm[r] : r;
        if ((unsigned)sr >= (unsigned)nrows) sr = r;
        dst[(size_t)r * dstride + doff + c] = src[(size_t)sr * C + c];
    }
}

template <typename T>
__global__ __launch_bounds__(256) void k_transpose_perm(const T *__restrict__ wd, int d, int f,
                                                        const int32_t *__restrict__ inv,
                                                        T *__restrict__ bundles, size_t bstride,
                                                        size_t doff) {
    __shared__ T tile[64][65];
    const int i0 = blockIdx.x * 64, m0 = blockIdx.y * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int r = ty; r < 64; r += 4) {
        const int m = m0 + r, i = i0 + tx;
        tile[r][tx] = (m < d && i < f) ? wd[(size_t)m * f + i] : T(0);
    }
    __syncthreads();
    for (int r = ty; r < 64; r += 4) {
        const int i = i0 + r, m = m0 + tx;
        if (i < f && m < d) {
            int s = inv[i];
            if ((unsigned)s >= (unsigned)f) s = i;
            bundles[(size_t)s * bstride + doff + m] = tile[tx][r];
        }
    }
}

__global__ void k_invert(const int32_t *__restrict__ perm, int f, int32_t *__restrict__ inv) {
    for (int s = blockIdx.x * blockDim.x + threadIdx.x; s < f; s += gridDim.x * blockDim.x) {
        int id = perm ? perm[s] : s;
        if ((unsigned)id < (unsigned)f) inv[id] = s;
    }
}

__global__ void k_fill_identity(int32_t *__restrict__ v, int n) {
    for (int s = blockIdx.x * blockDim.x + threadIdx.x; s < n; s += gridDim.x * blockDim.x) v[s] = s;
}

__global__ void k_gather_f32(const float *__restrict__ src, const int32_t *__restrict__ perm, int n,
                             float *__restrict__ dst) {
    for (int s = blockIdx.x * blockDim.x + threadIdx.x; s < n; s += gridDim.x * blockDim.x) {
        int id = perm ? perm[s] : s;
        if ((unsigned)id >= (unsigned)n) id = s;
        dst[s] = src ? src[id] : 0.0f;
    }
}

// ---------------------------------------------------------------- predictor
// One row of predictor layer 1, computed by one wave for every token:
// lane l holds chunks l, l+64, ... of the row; h[b][row] = max(0, sum + c1).
template <int WT, int CPL, int BT>
__device__ __forceinline__ void l1_row(const u32x4 *__restrict__ P1, const float *__restrict__ c1,
                                       const float *__restrict__ x, int B, int d, int H, int row,
                                       float *__restrict__ h, int lane) {
    constexpr int E = Elt<WT>::E;
    const int C = d / E;
    const u32x4 *prow = P1 + (size_t)row * C;
    u32x4 w[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = lane + 64 * i;
        w[i] = c < C ? prow[c] : u32x4{0u, 0u, 0u, 0u};
    }
    const float bias = c1[row];
    for (int b0 = 0; b0 < B; b0 += BT) {
        float acc[BT];
#pragma unroll
        for (int t = 0; t < BT; ++t) acc[t] = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + 64 * i;
            if (c < C) {
                float wv[E];
                unpack<WT>(w[i], wv);
#pragma unroll
                for (int t = 0; t < BT; ++t) {
                    if (BT == 1 || b0 + t < B) {
                        float xv[E];
                        load_f32<E>(x + (size_t)(b0 + t) * d + (size_t)c * E, xv);
#pragma unroll
                        for (int e = 0; e < E; ++e) acc[t] = fmaf(wv[e], xv[e], acc[t]);
                    }
                }
            }
        }
#pragma unroll
        for (int t = 0; t < BT; ++t) {
            const float s = wave_sum(acc[t]) + bias;
            if (lane == 0 && (BT == 1 || b0 + t < B)) h[(size_t)(b0 + t) * H + row] = fmaxf(s, 0.0f);
        }
    }
}

// Loads of the kL2Rows predictor layer-2 rows slot0 .. slot0+7 of one wave
// (lane l holds chunks l, l+64, ... of each row) and of their biases.
template <int CPL>
__device__ __forceinline__ void l2_load(const u32x4 *__restrict__ P2, const float *__restrict__ c2,
                                        int f, int C, int slot0, int lane,
                                        u32x4 (&w)[kL2Rows][CPL], float (&bias)[kL2Rows]) {
#pragma unroll
    for (int j = 0; j < kL2Rows; ++j) {
        const int slot = slot0 + j;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + 64 * i;
            w[j][i] = (slot < f && c < C) ? P2[(size_t)slot * C + c] : u32x4{0u, 0u, 0u, 0u};
        }
        bias[j] = slot < f ? c2[slot] : 0.0f;
    }
}

// Scores of those rows for tokens b0 .. b0+BT-1 against h; bit j of bits[t]
// is set when s(slot0 + j) > theta for token b0 + t.
template <int WT, int CPL, int BT>
__device__ __forceinline__ void l2_bits(const u32x4 (&w)[kL2Rows][CPL],
                                        const float (&bias)[kL2Rows], const float *__restrict__ h,
                                        int b0, int B, int H, int f, int slot0, float theta,
                                        int lane, uint32_t (&bits)[BT]) {
    constexpr int E = Elt<WT>::E;
    const int C = H / E;
    float hv[BT][CPL][E];
#pragma unroll
    for (int t = 0; t < BT; ++t)
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + 64 * i;
            if (c < C && (BT == 1 || b0 + t < B))
                load_f32<E>(h + (size_t)(b0 + t) * H + (size_t)c * E, hv[t][i]);
            else
#pragma unroll
                for (int e = 0; e < E; ++e) hv[t][i][e] = 0.0f;
        }
#pragma unroll
    for (int t = 0; t < BT; ++t) bits[t] = 0u;
#pragma unroll
    for (int j = 0; j < kL2Rows; ++j) {
        float acc[BT];
#pragma unroll
        for (int t = 0; t < BT; ++t) acc[t] = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            float wv[E];
            unpack<WT>(w[j][i], wv);
#pragma unroll
            for (int t = 0; t < BT; ++t)
#pragma unroll
                for (int e = 0; e < E; ++e) acc[t] = fmaf(wv[e], hv[t][i][e], acc[t]);
        }
#pragma unroll
        for (int t = 0; t < BT; ++t) {
            const float s = wave_sum(acc[t]) + bias[j];
            if (slot0 + j < f && s > theta) bits[t] |= 1u << j;
        }
    }
}

// Layer 1 as a kernel: one wave per hidden unit, 4 waves per workgroup.
template <int WT, int CPL, int BT>
__global__ __launch_bounds__(256) void k_pred_l1(const u32x4 *__restrict__ P1,
                                                 const float *__restrict__ c1,
                                                 const float *__restrict__ x, int B, int d, int H,
                                                 float *__restrict__ h) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= H) return;
    l1_row<WT, CPL, BT>(P1, c1, x, B, d, H, row, h, threadIdx.x & 63);
}

// Layer 2 + threshold as a kernel: workgroup = one 64-slot mask word, wave w
// scores slots 8w .. 8w+7 of it.
template <int WT, int CPL, int BT>
__global__ __launch_bounds__(kFfnThreads) void k_pred_l2(const u32x4 *__restrict__ P2,
                                                         const float *__restrict__ c2,
                                                         const float *__restrict__ h, int B, int H,
                                                         int f, int words, float theta,
                                                         uint64_t *__restrict__ masks) {
    constexpr int E = Elt<WT>::E;
    __shared__ uint32_t bits_lds[BT][kWaves];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int word = blockIdx.x;
    const int slot0 = word * 64 + wave * kL2Rows;
    u32x4 w[kL2Rows][CPL];
    float bias[kL2Rows];
    l2_load<CPL>(P2, c2, f, H / E, slot0, lane, w, bias);
    for (int b0 = 0; b0 < B; b0 += BT) {
        uint32_t bits[BT];
        l2_bits<WT, CPL, BT>(w, bias, h, b0, B, H, f, slot0, theta, lane, bits);
        if (lane == 0) {
#pragma unroll
            for (int t = 0; t < BT; ++t) bits_lds[t][wave] = bits[t];
        }
        __syncthreads();
        if (threadIdx.x < BT && (BT == 1 || b0 + (int)threadIdx.x < B)) {
            const int t = threadIdx.x;
            uint64_t m = 0;
#pragma unroll
            for (int q = 0; q < kWaves; ++q) m |= (uint64_t)bits_lds[t][q] << (kL2Rows * q);
            masks[(size_t)(b0 + t) * words + word] = m;
        }
        __syncthreads();
    }
}

// Compaction as a kernel: one workgroup of 1024 threads; thread t owns mask
// word t.  Union over the batch, popcount, exclusive prefix sum, then each
// thread writes its set bits in ascending slot order at its offset.
__global__ __launch_bounds__(1024) void k_compact(const uint64_t *__restrict__ masks, int B,
                                                  int words, const int32_t *__restrict__ perm,
                                                  uint64_t *__restrict__ umask,
                                                  int32_t *__restrict__ slots,
                                                  int32_t *__restrict__ count,
                                                  int32_t *__restrict__ active_ids,
                                                  int32_t *__restrict__ n_active) {
    __shared__ int wave_tot[16];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    uint64_t u = 0;
    if (t < words) {
        for (int b = 0; b < B; ++b) u |= masks[(size_t)b * words + t];
        umask[t] = u;
    }
    const int c = __popcll(u);
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int q = 0; q < wave; ++q) base += wave_tot[q];
    int off = base + incl - c;
    while (u) {
        const int j = __ffsll((unsigned long long)u) - 1;
        u &= u - 1;
        const int slot = t * 64 + j;
        slots[off] = slot;
        if (active_ids) active_ids[off] = perm[slot];
        ++off;
    }
    if (t == (int)blockDim.x - 1) {
        const int total = base + incl;
        *count = total;
        if (n_active) *n_active = total;
    }
}

// ---------------------------------------------------------------- FFN
// One workgroup's share of the FFN: the neurons at list positions g, g+G, ...
// (slot_of(q) gives the slot of the q-th of them, or -1 to skip).  Threads
// split each neuron's rows into 16-byte chunks (thread t owns chunks t,
// t+NT, ...).  Neurons go in batches of NB: all their chunk loads are issued,
// per-thread partial dots are reduced across the wave and then across the
// waves through LDS, and each thread adds a * down-column into the partial
// of y it owns.  The partial is written to partial_g [B][d].
template <int WT, bool GATED, int CPT, int BT, class SlotOf>
__device__ __forceinline__ void ffn_wg(const u32x4 *__restrict__ bundles,
                                       const float *__restrict__ b1, const float *__restrict__ x,
                                       int B, int d, int nmine, SlotOf slot_of,
                                       float *__restrict__ partial_g) {
    constexpr int E = Elt<WT>::E;
    constexpr int NMAT = GATED ? 3 : 2;
    constexpr int NB = (CPT * (GATED ? 3 : 2) * (BT > 1 ? 2 : 1) > 4) ? 4 : 8;
    constexpr int UP = GATED ? 1 : 0, DN = NMAT - 1;
    __shared__ float red[2][NB][BT][kWaves];

    const int tid = threadIdx.x, NT = blockDim.x, nw = NT >> 6, lane = tid & 63, wave = tid >> 6;
    const int C = d / E;
    const size_t bstride = (size_t)NMAT * C;

    for (int b0 = 0; b0 < B; b0 += BT) {
        float xv[BT][CPT][E], yacc[BT][CPT][E];
#pragma unroll
        for (int t = 0; t < BT; ++t)
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int c = tid + NT * i;
#pragma unroll
                for (int e = 0; e < E; ++e) yacc[t][i][e] = 0.0f;
                if (c < C && (BT == 1 || b0 + t < B))
                    load_f32<E>(x + (size_t)(b0 + t) * d + (size_t)c * E, xv[t][i]);
                else
#pragma unroll
                    for (int e = 0; e < E; ++e) xv[t][i][e] = 0.0f;
            }

        for (int q0 = 0; q0 < nmine; q0 += NB) {
            int slot[NB];
#pragma unroll
            for (int k = 0; k < NB; ++k) slot[k] = (q0 + k < nmine) ? slot_of(q0 + k) : -1;
            u32x4 wu[NB][CPT], wd[NB][CPT], wg[GATED ? NB : 1][CPT];
#pragma unroll
            for (int k = 0; k < NB; ++k)
#pragma unroll
                for (int i = 0; i < CPT; ++i) {
                    const int c = tid + NT * i;
                    const bool ok = slot[k] >= 0 && c < C;
                    const u32x4 *bp = bundles + (size_t)(ok ? slot[k] : 0) * bstride + c;
                    const u32x4 z = {0u, 0u, 0u, 0u};
                    wu[k][i] = ok ? bp[(size_t)UP * C] : z;
                    wd[k][i] = ok ? bp[(size_t)DN * C] : z;
                    if constexpr (GATED) wg[k][i] = ok ? bp[0] : z;
                }
            // partial dots
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                float pu[BT], pg[BT];
#pragma unroll
                for (int t = 0; t < BT; ++t) pu[t] = pg[t] = 0.0f;
#pragma unroll
                for (int i = 0; i < CPT; ++i) {
                    float vu[E];
                    unpack<WT>(wu[k][i], vu);
#pragma unroll
                    for (int t = 0; t < BT; ++t)
#pragma unroll
                        for (int e = 0; e < E; ++e) pu[t] = fmaf(vu[e], xv[t][i][e], pu[t]);
                    if constexpr (GATED) {
                        float vg[E];
                        unpack<WT>(wg[k][i], vg);
#pragma unroll
                        for (int t = 0; t < BT; ++t)
#pragma unroll
                            for (int e = 0; e < E; ++e) pg[t] = fmaf(vg[e], xv[t][i][e], pg[t]);
                    }
                }
#pragma unroll
                for (int t = 0; t < BT; ++t) {
                    const float su = wave_sum(pu[t]);
                    float sg = 0.0f;
                    if constexpr (GATED) sg = wave_sum(pg[t]);
                    if (lane == 0) {
                        red[0][k][t][wave] = su;
                        red[1][k][t][wave] = sg;
                    }
                }
            }
            __syncthreads();
            float a[NB][BT];
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                const float bias = slot[k] >= 0 ? b1[slot[k]] : 0.0f;
#pragma unroll
                for (int t = 0; t < BT; ++t) {
                    float su = 0.0f, sg = 0.0f;
                    for (int w = 0; w < nw; ++w) {
                        su += red[0][k][t][w];
                        if constexpr (GATED) sg += red[1][k][t][w];
                    }
                    float av;
                    if constexpr (GATED)
                        av = fmaxf(sg + bias, 0.0f) * su;
                    else
                        av = fmaxf(su + bias, 0.0f);
                    a[k][t] = slot[k] >= 0 ? av : 0.0f;
                }
            }
            __syncthreads();
            // AXPY of the down columns
#pragma unroll
            for (int k = 0; k < NB; ++k)
#pragma unroll
                for (int i = 0; i < CPT; ++i) {
                    float vd[E];
                    unpack<WT>(wd[k][i], vd);
#pragma unroll
                    for (int t = 0; t < BT; ++t)
#pragma unroll
                        for (int e = 0; e < E; ++e)
                            yacc[t][i][e] = fmaf(a[k][t], vd[e], yacc[t][i][e]);
                }
        }
        // this workgroup's partial of y
#pragma unroll
        for (int t = 0; t < BT; ++t)
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int c = tid + NT * i;
                if (c < C && (BT == 1 || b0 + t < B)) {
                    float4 *dst = reinterpret_cast<float4 *>(partial_g + (size_t)(b0 + t) * d +
                                                             (size_t)c * E);
#pragma unroll
                    for (int k = 0; k < E / 4; ++k)
                        dst[k] = make_float4(yacc[t][i][4 * k], yacc[t][i][4 * k + 1],
                                             yacc[t][i][4 * k + 2], yacc[t][i][4 * k + 3]);
                }
            }
    }
}

// FFN as a kernel over a list: list_mode 0 = slots, 1 = original ids (mapped
// through the inverse neuron table, out-of-range ids skipped), 2 = all slots.
template <int WT, bool GATED, int CPT, int BT>
__global__ __launch_bounds__(kFfnThreads) void k_ffn(
    const u32x4 *__restrict__ bundles, const float *__restrict__ b1, const float *__restrict__ x,
    int B, int d, int f, int list_mode, const int32_t *__restrict__ list,
    const int32_t *__restrict__ list_count, const int32_t *__restrict__ inv,
    float *__restrict__ partial) {
    const int G = gridDim.x, g = blockIdx.x;
    int n;
    if (list_mode == 2) {
        n = f;
    } else {
        n = *list_count;
        n = n < 0 ? 0 : (n > f ? f : n);
    }
    const int nmine = n > g ? (n - g + G - 1) / G : 0;
    auto slot_of = [&](int q) -> int {
        const int j = g + G * q;
        int s;
        if (list_mode == 2) {
            s = j;
        } else if (list_mode == 0) {
            s = list[j];
        } else {
            const int id = list[j];
            s = ((unsigned)id < (unsigned)f) ? inv[id] : -1;
        }
        return ((unsigned)s < (unsigned)f) ? s : -1;
    };
    ffn_wg<WT, GATED, CPT, BT>(bundles, b1, x, B, d, nmine, slot_of,
                               partial + (size_t)g * B * d);
}

// ---------------------------------------------------------------- reduction
// One tile of 32 outputs of one token: y[b][m] = (sum over workgroups g of
// partial[g][b][m]) + b2[m] + resid[b][m].  Threads 0..255 work (8 groups of
// 32; group q sums g = q, q+8, ... in ascending order), all threads of the
// workgroup must call it.
__device__ __forceinline__ void reduce_tile(const float *__restrict__ partial, int G, int B, int d,
                                            const float *__restrict__ b2, const float *resid,
                                            float *y, int tile, float (&red)[8][32]) {
    constexpr int KMAX = kFfnGroups / 8;
    const int tiles = (d + 31) / 32;
    const int b = tile / tiles, m = (tile % tiles) * 32 + (threadIdx.x & 31);
    const int grp = threadIdx.x >> 5;
    if (threadIdx.x < 256) {
        float v[KMAX];
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const int g = grp + 8 * k;
            v[k] = (g < G && m < d) ? partial[((size_t)g * B + b) * d + m] : 0.0f;
        }
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) acc += v[k];
        red[grp][threadIdx.x & 31] = acc;
    }
    __syncthreads();
    if (grp == 0 && m < d) {
        float s = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q) s += red[q][threadIdx.x];
        s += b2[m];
        if (resid) s += resid[(size_t)b * d + m];
        y[(size_t)b * d + m] = s;
    }
    __syncthreads();
}

__global__ __launch_bounds__(256) void k_reduce(const float *__restrict__ partial, int G, int B,
                                                int d, const float *__restrict__ b2,
                                                const float *resid, float *y) {
    __shared__ float red[8][32];
    reduce_tile(partial, G, B, d, b2, resid, y, blockIdx.x, red);
}

// ---------------------------------------------------------------- fused step
struct DecodeParams {
    const u32x4 *p1;
    const float *c1;
    const u32x4 *p2;
    const float *c2;
    const u32x4 *bundles;
    const float *b1;
    const float *b2;
    const int32_t *perm;
    int d, f, H, words;
    float theta;
    const float *x;
    const float *resid;
    float *y;
    float *h;
    uint64_t *masks;
    uint64_t *umask;
    int32_t *slots;
    int32_t *count;
    float *partial;
    unsigned *bar;
    int *err;
    int32_t *active_ids;
    int32_t *n_active;
};

// One decode step of one token (B = 1) in one cooperative launch of
// kFfnGroups workgroups x kFfnThreads threads.  Phases, split by grid
// barriers: (1) predictor layer 1, with the layer-2 rows of this workgroup's
// first mask word already in flight; (2) layer 2 + threshold -> mask words;
// (3) every workgroup rebuilds the prefix sums of the mask words in LDS,
// finds the slots at its list positions g, g+G, ... by binary search, writes
// them to the active list, and runs its FFN share; (4) reduction tiles.
template <int WT, int CPL1, int CPL2, bool GATED, int CPT>
__global__ __launch_bounds__(kFfnThreads) void k_decode(DecodeParams p) {
    constexpr int E = Elt<WT>::E;
    __shared__ uint64_t um[kMaxFfn / 64];
    __shared__ int pre[kMaxFfn / 64 + 1];
    __shared__ int wave_tot[kWaves];
    __shared__ uint32_t bits_lds[kWaves];
    __shared__ float red[8][32];
    __shared__ int myslots[kMaxFfn / kFfnGroups];

    const int G = gridDim.x, g = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int GW = G * kWaves, gw = g * kWaves + wave;

    // (0) layer-2 rows of the first word of this workgroup: loads in flight now
    u32x4 w2[kL2Rows][CPL2];
    float bias2[kL2Rows];
    const int C2 = p.H / E;
    if (g < p.words) l2_load<CPL2>(p.p2, p.c2, p.f, C2, g * 64 + wave * kL2Rows, lane, w2, bias2);

    // (1) predictor layer 1
    for (int row = gw; row < p.H; row += GW)
        l1_row<WT, CPL1, 1>(p.p1, p.c1, p.x, 1, p.d, p.H, row, p.h, lane);
    grid_sync(p.bar, G, p.err);

    // (2) layer 2 + threshold
    for (int q = g; q < p.words; q += G) {
        const int slot0 = q * 64 + wave * kL2Rows;
        if (q != g) l2_load<CPL2>(p.p2, p.c2, p.f, C2, slot0, lane, w2, bias2);
        uint32_t bits[1];
        l2_bits<WT, CPL2, 1>(w2, bias2, p.h, 0, 1, p.H, p.f, slot0, p.theta, lane, bits);
        if (lane == 0) bits_lds[wave] = bits[0];
        __syncthreads();
        if (tid == 0) {
            uint64_t m = 0;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) m |= (uint64_t)bits_lds[w] << (kL2Rows * w);
            p.masks[q] = m;
        }
        __syncthreads();
    }
    grid_sync(p.bar, G, p.err);

    // (3) compaction: prefix sums of the popcounts of all words (thread t owns
    // words 2t and 2t+1)
    const int w0 = 2 * tid;
    const uint64_t m0 = w0 < p.words ? p.masks[w0] : 0ull;
    const uint64_t m1 = w0 + 1 < p.words ? p.masks[w0 + 1] : 0ull;
    if (w0 < p.words) um[w0] = m0;
    if (w0 + 1 < p.words) um[w0 + 1] = m1;
    const int loc = __popcll(m0) + __popcll(m1);
    int incl = loc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int base = 0, total = 0;
    for (int w = 0; w < kWaves; ++w) {
        if (w < wave) base += wave_tot[w];
        total += wave_tot[w];
    }
    {
        const int ex = base + incl - loc;
        if (w0 < p.words) pre[w0] = ex;
        if (w0 + 1 < p.words) pre[w0 + 1] = ex + __popcll(m0);
    }
    __syncthreads();
    if (g == 0) {
        for (int w = tid; w < p.words; w += blockDim.x) p.umask[w] = um[w];
        if (tid == 0) {
            *p.count = total;
            if (p.n_active) *p.n_active = total;
        }
    }
    // slots of this workgroup's list positions j = g + G*q: thread q finds
    // the word holding the j-th set bit (binary search over the prefix sums)
    // and the bit inside it; the slots go to LDS and to the active list
    const int nmine = total > g ? (total - g + G - 1) / G : 0;
    if (tid < nmine) {
        const int j = g + G * tid;
        int lo = 0, hi = p.words - 1;  // last word w with pre[w] <= j
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (pre[mid] <= j) lo = mid;
            else hi = mid - 1;
        }
        uint64_t m = um[lo];
        int r = j - pre[lo], off = 0;
#pragma unroll
        for (int step = 32; step >= 8; step >>= 1) {
            const uint64_t low = m & ((1ull << step) - 1ull);
            const int c = __popcll(low);
            if (r >= c) {
                r -= c;
                m >>= step;
                off += step;
            } else {
                m = low;
            }
        }
        for (; r > 0; --r) m &= m - 1;
        const int s = lo * 64 + off + __ffsll((unsigned long long)m) - 1;
        myslots[tid] = s;
        p.slots[j] = s;
        if (p.active_ids) p.active_ids[j] = p.perm[s];
    }
    __syncthreads();
    auto slot_of = [&](int q) -> int { return myslots[q]; };
    ffn_wg<WT, GATED, CPT, 1>(p.bundles, p.b1, p.x, 1, p.d, nmine, slot_of,
                              p.partial + (size_t)g * p.d);
    grid_sync(p.bar, G, p.err);

    // (4) reduction
    const int tiles = (p.d + 31) / 32;
    for (int t = g; t < tiles; t += G) reduce_tile(p.partial, G, 1, p.d, p.b2, p.resid, p.y, t, red);
}

__global__ void k_read_error(int *err, int32_t *out, int clear) {
    if (threadIdx.x == 0) {
        *out = *err;
        if (clear) *err = 0;
    }
}

inline void trace_mark(const Trace *tr, int k, int edge, hipStream_t s) {
    if (tr && tr->ev[2 * k + edge]) (void)hipEventRecord(tr->ev[2 * k + edge], s);
}

inline int pow2_at_least(int v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

}  // namespace

// ================================================================ launchers
hipError_t launch_perm_rows(const void *src, int C, const int32_t *perm, int nrows, void *dst,
                            size_t dstride, size_t doff, hipStream_t s) {
    const size_t total = (size_t)nrows * C;
    const int blocks = (int)((total + 255) / 256 < 8192 ? (total + 255) / 256 : 8192);
    hipLaunchKernelGGL(k_perm_rows, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, s,
                       (const u32x4 *)src, C, perm, nrows, (u32x4 *)dst, dstride, doff);
    return hipGetLastError();
}

hipError_t launch_transpose_perm(const void *wd, int d, int f, int ws, const int32_t *inv,
                                 void *bundles, size_t bstride, size_t doff, hipStream_t s) {
    dim3 grid((f + 63) / 64, (d + 63) / 64);
    if (ws == 2)
        hipLaunchKernelGGL(k_transpose_perm<uint16_t>, grid, dim3(256), 0, s, (const uint16_t *)wd,
                           d, f, inv, (uint16_t *)bundles, bstride, doff);
    else
        hipLaunchKernelGGL(k_transpose_perm<uint32_t>, grid, dim3(256), 0, s, (const uint32_t *)wd,
                           d, f, inv, (uint32_t *)bundles, bstride, doff);
    return hipGetLastError();
}

hipError_t launch_invert(const int32_t *perm, int f, int32_t *inv, hipStream_t s) {
    const int blocks = (f + 255) / 256;
    hipLaunchKernelGGL(k_fill_identity, dim3(blocks), dim3(256), 0, s, inv, f);
    hipLaunchKernelGGL(k_invert, dim3(blocks), dim3(256), 0, s, perm, f, inv);
    return hipGetLastError();
}

hipError_t launch_gather_f32(const float *src, const int32_t *perm, int n, float *dst,
                             hipStream_t s) {
    hipLaunchKernelGGL(k_gather_f32, dim3((n + 255) / 256), dim3(256), 0, s, src, perm, n, dst);
    return hipGetLastError();
}

template <int WT>
static void dispatch_pred(const LayerView &L, const float *x, int B, uint64_t *masks,
                          const Trace *tr, hipStream_t s) {
    const int cpl1 = pow2_at_least((L.cd + 63) / 64);
    const dim3 g1((L.H + 3) / 4), blk(256);
    const u32x4 *P1 = (const u32x4 *)L.p1;
#define ASF_L1(CPL, BT) \
    hipLaunchKernelGGL((k_pred_l1<WT, CPL, BT>), g1, blk, 0, s, P1, L.c1, x, B, L.d, L.H, L.h)
#define ASF_L1B(CPL) \
    if (B == 1) ASF_L1(CPL, 1); else ASF_L1(CPL, 4);
    trace_mark(tr, ASF_K_PRED_L1, 0, s);
    switch (cpl1) {
    case 1: ASF_L1B(1) break;
    case 2: ASF_L1B(2) break;
    case 4: ASF_L1B(4) break;
    case 8: ASF_L1B(8) break;
    default: ASF_L1B(16) break;
    }
    trace_mark(tr, ASF_K_PRED_L1, 1, s);
#undef ASF_L1B
#undef ASF_L1
    const int cpl2 = pow2_at_least((L.ch + 63) / 64);
    const dim3 g2(L.words), blk2(kFfnThreads);
    const u32x4 *P2 = (const u32x4 *)L.p2;
#define ASF_L2(CPL, BT)                                                                        \
    hipLaunchKernelGGL((k_pred_l2<WT, CPL, BT>), g2, blk2, 0, s, P2, L.c2, L.h, B, L.H, L.f, \
                       L.words, L.threshold, masks)
#define ASF_L2B(CPL) \
    if (B == 1) ASF_L2(CPL, 1); else ASF_L2(CPL, 4);
    trace_mark(tr, ASF_K_PRED_L2, 0, s);
    switch (cpl2) {
    case 1: ASF_L2B(1) break;
    case 2: ASF_L2B(2) break;
    default: ASF_L2B(4) break;
    }
    trace_mark(tr, ASF_K_PRED_L2, 1, s);
#undef ASF_L2B
#undef ASF_L2
}

hipError_t launch_predict(const LayerView &L, const float *x, int B, int32_t *active_ids,
                          int32_t *n_active, uint64_t *token_masks, const Trace *tr,
                          hipStream_t s) {
    uint64_t *masks = token_masks ? token_masks : L.masks;
    if (L.wtype == ASF_F16)
        dispatch_pred<1>(L, x, B, masks, tr, s);
    else
        dispatch_pred<0>(L, x, B, masks, tr, s);
    trace_mark(tr, ASF_K_COMPACT, 0, s);
    hipLaunchKernelGGL(k_compact, dim3(1), dim3(1024), 0, s, (const uint64_t *)masks, B, L.words,
                       (const int32_t *)L.perm, L.umask, L.slots, L.count, active_ids, n_active);
    trace_mark(tr, ASF_K_COMPACT, 1, s);
    return hipGetLastError();
}

template <int WT, bool GATED>
static void dispatch_ffn(const LayerView &L, const float *x, int B, int list_mode,
                         const int32_t *list, const int32_t *cnt, hipStream_t s) {
    constexpr int E = WT ? 8 : 4;
    const int C = L.d / E;
    const int cpt = (C + kFfnThreads - 1) / kFfnThreads;
    const u32x4 *bp = (const u32x4 *)L.bundles;
#define ASF_FFN(CPT, BT)                                                                     \
    hipLaunchKernelGGL((k_ffn<WT, GATED, CPT, BT>), dim3(kFfnGroups), dim3(kFfnThreads), 0, \
                       s, bp, L.b1, x, B, L.d, L.f, list_mode, list, cnt, L.inv,           \
                       L.partial)
    if (cpt <= 1) {
        if (B == 1) ASF_FFN(1, 1); else ASF_FFN(1, 4);
    } else {
        if (B == 1) ASF_FFN(2, 1); else ASF_FFN(2, 4);
    }
#undef ASF_FFN
}

hipError_t launch_ffn(const LayerView &L, const float *x, int B, int list_mode, const int32_t *ids,
                      const int32_t *n_ids, const float *resid, float *y, const Trace *tr,
                      hipStream_t s) {
    const int32_t *list = list_mode == 0 ? L.slots : ids;
    const int32_t *cnt = list_mode == 0 ? L.count : n_ids;
    trace_mark(tr, ASF_K_FFN, 0, s);
    if (L.wtype == ASF_F16) {
        if (L.gated) dispatch_ffn<1, true>(L, x, B, list_mode, list, cnt, s);
        else dispatch_ffn<1, false>(L, x, B, list_mode, list, cnt, s);
    } else {
        if (L.gated) dispatch_ffn<0, true>(L, x, B, list_mode, list, cnt, s);
        else dispatch_ffn<0, false>(L, x, B, list_mode, list, cnt, s);
    }
    trace_mark(tr, ASF_K_FFN, 1, s);
    const int tiles = (L.d + 31) / 32;
    trace_mark(tr, ASF_K_REDUCE, 0, s);
    hipLaunchKernelGGL(k_reduce, dim3(B * tiles), dim3(256), 0, s, (const float *)L.partial,
                       kFfnGroups, B, L.d, (const float *)L.b2, resid, y);
    trace_mark(tr, ASF_K_REDUCE, 1, s);
    return hipGetLastError();
}

// ---------------------------------------------------------------- fused step
// Kernel pointer of the fused decode kernel for a layer, or null when the
// layer's shape has no fused variant (fp32 weights).
static const void *decode_kernel(const LayerView &L) {
    if (L.wtype != ASF_F16) return nullptr;
    const int cpl1 = pow2_at_least((L.cd + 63) / 64);
    const int cpl2 = pow2_at_least((L.ch + 63) / 64);
    const int cpt = (L.cd + kFfnThreads - 1) / kFfnThreads;
    if (cpl1 < 4 || cpl1 > 16 || cpl2 > 4 || cpt > 2) return nullptr;
#define ASF_DK(C1, C2, CT)                                                                  \
    return L.gated ? (const void *)&k_decode<1, C1, C2, true, CT>                         \
                   : (const void *)&k_decode<1, C1, C2, false, CT>;
#define ASF_DK2(C1, CT)              \
    switch (cpl2) {                  \
    case 1: ASF_DK(C1, 1, CT)        \
    case 2: ASF_DK(C1, 2, CT)        \
    default: ASF_DK(C1, 4, CT)       \
    }
    if (cpl1 == 4) { ASF_DK2(4, 1) }
    if (cpl1 == 8) { ASF_DK2(8, 1) }
    ASF_DK2(16, 2)
#undef ASF_DK2
#undef ASF_DK
}

bool fused_supported(const LayerView &L) {
    const void *k = decode_kernel(L);
    if (!k) return false;
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return false;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kFfnThreads, 0) != hipSuccess)
        return false;
    return (long)per_cu * cus >= kFfnGroups;
}

hipError_t launch_decode_fused(const LayerView &L, const float *x, const float *resid, float *y,
                               int32_t *active_ids, int32_t *n_active, const Trace *tr,
                               hipStream_t s) {
    const void *k = decode_kernel(L);
    if (!k) return hipErrorInvalidValue;
    DecodeParams p;
    p.p1 = (const u32x4 *)L.p1;
    p.c1 = L.c1;
    p.p2 = (const u32x4 *)L.p2;
    p.c2 = L.c2;
    p.bundles = (const u32x4 *)L.bundles;
    p.b1 = L.b1;
    p.b2 = L.b2;
    p.perm = L.perm;
    p.d = L.d;
    p.f = L.f;
    p.H = L.H;
    p.words = L.words;
    p.theta = L.threshold;
    p.x = x;
    p.resid = resid;
    p.y = y;
    p.h = L.h;
    p.masks = L.masks;
    p.umask = L.umask;
    p.slots = L.slots;
    p.count = L.count;
    p.partial = L.partial;
    p.bar = L.bar;
    p.err = L.err;
    p.active_ids = active_ids;
    p.n_active = n_active;
    void *args[] = {&p};
    trace_mark(tr, ASF_K_DECODE, 0, s);
    hipError_t e = hipLaunchCooperativeKernel(k, dim3(kFfnGroups), dim3(kFfnThreads), args, 0, s);
    trace_mark(tr, ASF_K_DECODE, 1, s);
    return e != hipSuccess ? e : hipGetLastError();
}

hipError_t launch_read_error(const LayerView &L, int32_t *out, int clear, hipStream_t s) {
    hipLaunchKernelGGL(k_read_error, dim3(1), dim3(64), 0, s, L.err, out, clear);
    return hipGetLastError();
}

}  // namespace asf
