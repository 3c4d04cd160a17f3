// asf_kernels.hip -- gfx950 kernels of the activation-sparse FFN decode path.
//
// Per decode step of one layer:
//   pred_l1   h = ReLU(P1 x + c1)                       dense GEMV, one wave per row
//   pred_l2   s = P2 h + c2, bit = s > theta           dense GEMV over slot-ordered
//             rows; 64 rows -> one uint64 mask word      rows of P2
//   compact   union of the tokens' masks, popcount + workgroup prefix sum ->
//             ascending slot list (and original ids through the neuron table)
//   ffn       per active neuron: FC1 dot of its up row with x (+b1, ReLU; or the
//             ReLU-gated form), then AXPY of its down column into y.  Each
//             workgroup owns a float32 partial of y.
//   reduce    y = residual + b2 + sum of the partials, in a fixed order.
//
// All weight reads are whole 16-byte chunks (64 lanes x 16 B = 1 KiB per wave
// instruction) of contiguous neuron rows: an active neuron's up row and down
// column sit back to back in one bundle, so its bytes form one contiguous run
// ("LLM模型之PowerInfer1.0", "其他" question 3: contiguous loads of active
// columns of the down projection, skipping the inactive ones).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "asf_internal.h"

namespace asf {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

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
// Layer 1: one wave per hidden unit k; lane l holds chunks l, l+64, ... of row k.
template <int WT, int CPL, int BT>
__global__ __launch_bounds__(256) void k_pred_l1(const u32x4 *__restrict__ P1,
                                                 const float *__restrict__ c1,
                                                 const float *__restrict__ x, int B, int d, int H,
                                                 float *__restrict__ h) {
    constexpr int E = Elt<WT>::E;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= H) return;
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

// Layer 2 + threshold: workgroup = one 64-slot mask word, wave w scores slots
// 16w .. 16w+15 of the word, one row at a time (all 16 rows' loads issued up
// front).  Bit j of word q is set when s(slot 64q+j) > theta.
template <int WT, int CPL, int BT>
__global__ __launch_bounds__(256) void k_pred_l2(const u32x4 *__restrict__ P2,
                                                 const float *__restrict__ c2,
                                                 const float *__restrict__ h, int B, int H, int f,
                                                 int words, float theta,
                                                 uint64_t *__restrict__ masks) {
    constexpr int E = Elt<WT>::E;
    constexpr int R = 16;
    __shared__ uint32_t bits_lds[BT][4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int word = blockIdx.x;
    const int C = H / E;
    const int slot0 = word * 64 + wave * R;
    u32x4 w[R][CPL];
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int slot = slot0 + j;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + 64 * i;
            w[j][i] = (slot < f && c < C) ? P2[(size_t)slot * C + c] : u32x4{0u, 0u, 0u, 0u};
        }
    }
    float bias[R];
#pragma unroll
    for (int j = 0; j < R; ++j) bias[j] = (slot0 + j < f) ? c2[slot0 + j] : 0.0f;

    for (int b0 = 0; b0 < B; b0 += BT) {
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
        uint32_t bits[BT];
#pragma unroll
        for (int t = 0; t < BT; ++t) bits[t] = 0u;
#pragma unroll
        for (int j = 0; j < R; ++j) {
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
        if (lane == 0) {
#pragma unroll
            for (int t = 0; t < BT; ++t) bits_lds[t][wave] = bits[t];
        }
        __syncthreads();
        if (threadIdx.x < BT && (BT == 1 || b0 + (int)threadIdx.x < B)) {
            const int t = threadIdx.x;
            uint64_t m = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) m |= (uint64_t)bits_lds[t][q] << (16 * q);
            masks[(size_t)(b0 + t) * words + word] = m;
        }
        __syncthreads();
    }
}

// Compaction: one workgroup of 1024 threads; thread t owns mask word t.
// Union over the batch, popcount, exclusive prefix sum, then each thread
// writes its set bits in ascending slot order at its offset.
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
// Workgroup g handles the neurons at list positions g, g+G, g+2G, ... (G =
// gridDim.x); its threads split each neuron's rows into 16-byte chunks
// (thread t owns chunks t, t+NT, ...).  Neurons go in batches of NB: all
// their chunk loads are issued, per-thread partial dots are reduced across
// the wave and then across the waves through LDS, and each thread adds
// a * down-column into the partial of y it owns for its chunks.
template <int WT, bool GATED, int CPT, int BT>
__global__ __launch_bounds__(kFfnThreads) void k_ffn(
    const u32x4 *__restrict__ bundles, const float *__restrict__ b1, const float *__restrict__ x,
    int B, int d, int f, int list_mode, const int32_t *__restrict__ list,
    const int32_t *__restrict__ list_count, const int32_t *__restrict__ inv,
    float *__restrict__ partial) {
    constexpr int E = Elt<WT>::E;
    constexpr int NMAT = GATED ? 3 : 2;
    constexpr int NB = (CPT * (GATED ? 3 : 2) * (BT > 1 ? 2 : 1) > 4) ? 4 : 8;
    constexpr int UP = GATED ? 1 : 0, DN = NMAT - 1;
    constexpr int NWMAX = kFfnThreads / 64;
    __shared__ float red[2][NB][BT][NWMAX];

    const int tid = threadIdx.x, NT = blockDim.x, nw = NT >> 6, lane = tid & 63, wave = tid >> 6;
    const int G = gridDim.x, g = blockIdx.x;
    const int C = d / E;
    const size_t bstride = (size_t)NMAT * C;
    int n;
    if (list_mode == 2) {
        n = f;
    } else {
        n = *list_count;
        n = n < 0 ? 0 : (n > f ? f : n);
    }
    const int nmine = n > g ? (n - g + G - 1) / G : 0;

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
            for (int k = 0; k < NB; ++k) {
                int s = -1;
                if (q0 + k < nmine) {
                    const int j = g + G * (q0 + k);
                    if (list_mode == 2) {
                        s = j;
                    } else if (list_mode == 0) {
                        s = list[j];
                    } else {
                        const int id = list[j];
                        s = ((unsigned)id < (unsigned)f) ? inv[id] : -1;
                    }
                    if ((unsigned)s >= (unsigned)f) s = -1;
                }
                slot[k] = s;
            }
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
                    float4 *dst = reinterpret_cast<float4 *>(
                        partial + ((size_t)g * B + b0 + t) * d + (size_t)c * E);
#pragma unroll
                    for (int k = 0; k < E / 4; ++k)
                        dst[k] = make_float4(yacc[t][i][4 * k], yacc[t][i][4 * k + 1],
                                             yacc[t][i][4 * k + 2], yacc[t][i][4 * k + 3]);
                }
            }
    }
}

// y[b][m] = (sum over groups g of partial[g][b][m]) + b2[m] + resid[b][m].
// Workgroup = 32 outputs of one token; 8 thread groups split the partials.
__global__ __launch_bounds__(256) void k_reduce(const float *__restrict__ partial, int G, int B,
                                                int d, const float *__restrict__ b2,
                                                const float *resid, float *y) {
    __shared__ float red[8][32];
    const int tiles = (d + 31) / 32;
    const int b = blockIdx.x / tiles, m = (blockIdx.x % tiles) * 32 + (threadIdx.x & 31);
    const int grp = threadIdx.x >> 5;
    float acc = 0.0f;
    if (m < d)
        for (int g = grp; g < G; g += 8) acc += partial[((size_t)g * B + b) * d + m];
    red[grp][threadIdx.x & 31] = acc;
    __syncthreads();
    if (grp == 0 && m < d) {
        float s = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q) s += red[q][threadIdx.x];
        s += b2[m];
        if (resid) s += resid[(size_t)b * d + m];
        y[(size_t)b * d + m] = s;
    }
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
                          hipStream_t s) {
    const int cpl1 = pow2_at_least((L.cd + 63) / 64);
    const dim3 g1((L.H + 3) / 4), blk(256);
    const u32x4 *P1 = (const u32x4 *)L.p1;
#define ASF_L1(CPL, BT) \
    hipLaunchKernelGGL((k_pred_l1<WT, CPL, BT>), g1, blk, 0, s, P1, L.c1, x, B, L.d, L.H, L.h)
#define ASF_L1B(CPL) \
    if (B == 1) ASF_L1(CPL, 1); else ASF_L1(CPL, 4);
    switch (cpl1) {
    case 1: ASF_L1B(1) break;
    case 2: ASF_L1B(2) break;
    case 4: ASF_L1B(4) break;
    case 8: ASF_L1B(8) break;
    default: ASF_L1B(16) break;
    }
#undef ASF_L1B
#undef ASF_L1
    const int cpl2 = pow2_at_least((L.ch + 63) / 64);
    const dim3 g2(L.words);
    const u32x4 *P2 = (const u32x4 *)L.p2;
#define ASF_L2(CPL, BT)                                                                       \
    hipLaunchKernelGGL((k_pred_l2<WT, CPL, BT>), g2, blk, 0, s, P2, L.c2, L.h, B, L.H, L.f, \
                       L.words, L.threshold, masks)
#define ASF_L2B(CPL) \
    if (B == 1) ASF_L2(CPL, 1); else ASF_L2(CPL, 4);
    switch (cpl2) {
    case 1: ASF_L2B(1) break;
    case 2: ASF_L2B(2) break;
    default: ASF_L2B(4) break;
    }
#undef ASF_L2B
#undef ASF_L2
}

hipError_t launch_predict(const LayerView &L, const float *x, int B, int32_t *active_ids,
                          int32_t *n_active, uint64_t *token_masks, hipStream_t s) {
    uint64_t *masks = token_masks ? token_masks : L.masks;
    if (L.wtype == ASF_F16)
        dispatch_pred<1>(L, x, B, masks, s);
    else
        dispatch_pred<0>(L, x, B, masks, s);
    hipLaunchKernelGGL(k_compact, dim3(1), dim3(1024), 0, s, (const uint64_t *)masks, B, L.words,
                       (const int32_t *)L.perm, L.umask, L.slots, L.count, active_ids, n_active);
    return hipGetLastError();
}

template <int WT, bool GATED>
static void dispatch_ffn(const LayerView &L, const float *x, int B, int list_mode,
                         const int32_t *list, const int32_t *cnt, hipStream_t s) {
    constexpr int E = WT ? 8 : 4;
    const int C = L.d / E;
    int nt = C >= kFfnThreads ? kFfnThreads : ((C + 63) / 64) * 64;
    const int cpt = (C + nt - 1) / nt;
    const u32x4 *bp = (const u32x4 *)L.bundles;
#define ASF_FFN(CPT, BT)                                                                     \
    hipLaunchKernelGGL((k_ffn<WT, GATED, CPT, BT>), dim3(kFfnGroups), dim3(nt), 0, s, bp, \
                       L.b1, x, B, L.d, L.f, list_mode, list, cnt, L.inv, L.partial)
    if (cpt <= 1) {
        if (B == 1) ASF_FFN(1, 1); else ASF_FFN(1, 4);
    } else {
        if (B == 1) ASF_FFN(2, 1); else ASF_FFN(2, 4);
    }
#undef ASF_FFN
}

hipError_t launch_ffn(const LayerView &L, const float *x, int B, int list_mode, const int32_t *ids,
                      const int32_t *n_ids, const float *resid, float *y, hipStream_t s) {
    const int32_t *list = list_mode == 0 ? L.slots : ids;
    const int32_t *cnt = list_mode == 0 ? L.count : n_ids;
    if (L.wtype == ASF_F16) {
        if (L.gated) dispatch_ffn<1, true>(L, x, B, list_mode, list, cnt, s);
        else dispatch_ffn<1, false>(L, x, B, list_mode, list, cnt, s);
    } else {
        if (L.gated) dispatch_ffn<0, true>(L, x, B, list_mode, list, cnt, s);
        else dispatch_ffn<0, false>(L, x, B, list_mode, list, cnt, s);
    }
    const int tiles = (L.d + 31) / 32;
    hipLaunchKernelGGL(k_reduce, dim3(B * tiles), dim3(256), 0, s, (const float *)L.partial,
                       kFfnGroups, B, L.d, (const float *)L.b2, resid, y);
    return hipGetLastError();
}

}  // namespace asf
