// asf_api.hip -- host side of the C ABI declared in include/asf.h: argument
// validation, carving of the caller's storage, the create-time layout pass
// (hot-first permutation of neuron rows, neuron-major down projection) and
// launch sequencing.  No device memory is allocated here.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <new>

#include "asf_internal.h"

namespace asf {

static inline uintptr_t align_up(uintptr_t v, uintptr_t a) { return (v + a - 1) & ~(a - 1); }

static bool desc_ok(const asf_layer_desc &d) {
    if (d.d_model <= 0 || d.d_ffn <= 0 || d.pred_hidden <= 0) return false;
    if (d.max_batch < 1 || d.max_batch > kMaxBatch) return false;
    if (d.d_ffn > kMaxFfn) return false;
    if (d.gated != 0 && d.gated != 1) return false;
    if (d.wtype != ASF_F32 && d.wtype != ASF_F16) return false;
    const int ws = d.wtype == ASF_F16 ? 2 : 4;
    if ((d.pred_hidden * ws) % 16 != 0) return false;
    // FC2 splits d into kSlices slices of whole 16-byte chunks
    if ((d.d_model * ws) % (16 * kSlices) != 0) return false;
    // register tiling limits: 16 chunks per lane for a d row, 4 for an H row
    const int cd = d.d_model * ws / 16, ch = d.pred_hidden * ws / 16;
    if (cd > 1024 || ch > 256) return false;
    return true;
}

size_t carve(const asf_layer_desc &desc, uintptr_t base, LayerView *v) {
    const int ws = desc.wtype == ASF_F16 ? 2 : 4;
    const size_t d = desc.d_model, f = desc.d_ffn, H = desc.pred_hidden, Bm = desc.max_batch;
    const int nmat = desc.gated ? 3 : 2;
    const size_t words = (f + 63) / 64, nq = words;
    uintptr_t p = align_up(base, 256);
    auto take = [&](size_t bytes) {
        uintptr_t q = p;
        p = align_up(p + bytes, 256);
        return q;
    };
    LayerView t;
    t.d = (int)d;
    t.f = (int)f;
    t.H = (int)H;
    t.max_batch = (int)Bm;
    t.gated = desc.gated;
    t.wtype = desc.wtype;
    t.threshold = desc.threshold;
    t.ws = ws;
    t.cd = (int)(d * ws / 16);
    t.ch = (int)(H * ws / 16);
    t.words = (int)words;
    t.nq = (int)nq;
    t.nmat = nmat;
    t.p1 = (void *)take(H * d * ws);
    t.c1 = (float *)take(H * 4);
    // owner-major rows (batched forms), padded to nq*64; k-major owner blocks
    // (one token)
    t.p2 = Bm > 1 ? (void *)take(nq * kRowsPerWG * H * ws) : nullptr;
    t.p2k = (void *)take(nq * kRowsPerWG * H * ws);
    t.c2 = (float *)take(f * 4);
    t.bundles = (void *)take(f * nmat * d * ws);
    t.b1 = (float *)take(f * 4);
    t.b2 = (float *)take(d * 4);
    t.perm = (int32_t *)take(f * 4);
    t.inv = (int32_t *)take(f * 4);
    t.h = (float *)take(Bm * H * 4);
    t.h16 = Bm > 1 ? (_Float16 *)take(2 * Bm * H * 2) : nullptr;
    t.x16 = Bm > 1 ? (_Float16 *)take(2 * Bm * (size_t)x16_pitch((int)d) * 2) : nullptr;
    t.wbits = (uint64_t *)take(Bm * nq * 8);
    t.ubits = (uint64_t *)take(nq * 8);
    t.vbits = (uint64_t *)take(nq * 8);
    t.lslot = (int32_t *)take(nq * kRowsPerWG * 4);
    t.la = (float *)take(nq * kRowsPerWG * Bm * 4);
    t.la16 = Bm > 1 ? (_Float16 *)take(2 * Bm * nq * kRowsPerWG * 2) : nullptr;
    t.fc1_part = Bm > 1 ? (float *)take((size_t)fc1_slices((int)d) * (nmat - 1) * Bm * nq *
                                        kRowsPerWG * 4)
                        : nullptr;
    t.partial = (float *)take((size_t)kGroups * Bm * d * 4);
    t.part1 = (float *)take(nq * d * 4);
    t.arrive = (unsigned *)take(kArrive * 4);
    // batched predictor partial tiles (row tiles x up to 8 k-splits x 32x32)
    t.pred_part = Bm > 1 ? (float *)take((size_t)pred_slices((int)d) * Bm * H * 4) : nullptr;
    t.masks = (uint64_t *)take(Bm * words * 8);
    t.slots = (int32_t *)take(f * 4);
    t.count = (int32_t *)take(64);
    t.rows = (int32_t *)take(64);
    t.dbg = (unsigned *)take(64);
    t.xstride = (int)H + 64;
    t.xch = (uint64_t *)take((size_t)kXchCopies * t.xstride * 8);
    t.epoch = (unsigned *)take(64);
    t.fused = 0;
    if (v) *v = t;
    return (size_t)(p - align_up(base, 256));
}

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

#ifdef ASF_DEBUG
// Debug builds: the caller's device content checked before use (ids in
// range and distinct, count in 0 .. f); synchronises the stream.  The
// layer's slot-ordered mask scratch (at least f bits) holds the bitmap.
static asf_status debug_check_ids(const LayerView &v, const int32_t *ids, const int32_t *n_ids,
                                  int n_fixed, hipStream_t s) {
    unsigned flags = 0;
    if (launch_check_ids(ids, n_ids, n_fixed, v.f, (uint32_t *)v.masks, v.dbg, s) != hipSuccess ||
        hipMemcpyAsync(&flags, v.dbg, 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return ASF_ERR_HIP;
    return flags ? ASF_ERR_ARG : ASF_OK;
}
#endif

static bool head_desc_ok(const asf_head_desc &d) {
    if (d.d_model <= 0 || d.n_heads <= 0 || d.pred_hidden <= 0) return false;
    if (d.n_heads > kMaxHeads || d.max_batch < 1 || d.max_batch > kMaxBatch) return false;
    if (d.wtype != ASF_F32 && d.wtype != ASF_F16) return false;
    const int ws = d.wtype == ASF_F16 ? 2 : 4;
    // layer 1 runs on the FFN predictor's kernels: the same row alignment
    if ((d.d_model * ws) % (16 * kSlices) != 0 || (d.pred_hidden * ws) % 16 != 0) return false;
    return d.d_model * ws / 16 <= 1024 && d.pred_hidden * ws / 16 <= 256;
}

size_t carve_heads(const asf_head_desc &desc, uintptr_t base, HeadView *v) {
    const int ws = desc.wtype == ASF_F16 ? 2 : 4;
    const size_t d = desc.d_model, nh = desc.n_heads, H = desc.pred_hidden,
                 Bm = desc.max_batch, words = (nh + 63) / 64;
    uintptr_t p = align_up(base, 256);
    auto take = [&](size_t bytes) {
        uintptr_t q = p;
        p = align_up(p + bytes, 256);
        return q;
    };
    HeadView t;
    t.d = (int)d;
    t.nh = (int)nh;
    t.H = (int)H;
    t.max_batch = (int)Bm;
    t.wtype = desc.wtype;
    t.threshold = desc.threshold;
    t.ws = ws;
    t.cd = (int)(d * ws / 16);
    t.ch = (int)(H * ws / 16);
    t.words = (int)words;
    t.q1 = (void *)take(H * d * ws);
    t.c1 = (float *)take(H * 4);
    t.q2 = (void *)take(nh * H * ws);
    t.c2 = (float *)take(nh * 4);
    t.h = (float *)take(Bm * H * 4);
    t.wbits = (uint64_t *)take(Bm * words * 8);
    t.h16 = Bm > 1 ? (_Float16 *)take(2 * Bm * H * 2) : nullptr;
    t.x16 = Bm > 1 ? (_Float16 *)take(2 * Bm * (size_t)x16_pitch((int)d) * 2) : nullptr;
    t.pred_part = Bm > 1 ? (float *)take((size_t)pred_slices((int)d) * Bm * H * 4) : nullptr;
    if (v) *v = t;
    return (size_t)(p - align_up(base, 256));
}

// FC2 after launch_score with FC1: a single token's owner rows are already
// formed (launch_fc2_sum adds them); batches go through the owner lists
static hipError_t launch_fc2_step(const LayerView &v, int B, const float *resid, float *y,
                                  const Trace *tr, hipStream_t s) {
    if (B == 1) return launch_fc2_sum(v, resid, y, tr, s);
    return launch_fc2(v, B, false, resid, y, tr, s);
}

// One decode step of layer v (predict, FC1, FC2 into y): one token in one
// launch when every owner can be resident at once (then the owner-row sum,
// which also advances the exchange epoch), else predictor layer 1, the
// scores with FC1, and FC2.  With active / n_active, the list of the step's
// set too: for one token in the owner-row sum's grid, else by the list
// kernel.
static hipError_t launch_step(const LayerView &v, const float *x, int B, const float *resid,
                              float *y, int32_t *active, int32_t *n_active, const Trace *tr,
                              hipStream_t s) {
    hipError_t e;
    const bool list = active || n_active;
    if (B == 1 && v.fused) {
        if ((e = launch_step1(v, x, tr, s)) != hipSuccess) return e;
        if (list) return launch_fc2_sum_list(v, resid, y, active, n_active, tr, s, true);
        return launch_fc2_sum(v, resid, y, tr, s, true);
    }
    if ((e = launch_pred_l1(v, x, B, tr, s)) != hipSuccess) return e;
    if ((e = launch_score(v, x, B, true, tr, s)) != hipSuccess) return e;
    if (B == 1 && list) return launch_fc2_sum_list(v, resid, y, active, n_active, tr, s, false);
    if ((e = launch_fc2_step(v, B, resid, y, tr, s)) != hipSuccess) return e;
    if (list) return launch_list(v, B, active, n_active, nullptr, tr, s);
    return hipSuccess;
}

// Inter-layer buffer of asf_stack_decode_static: one [B][d_model] float32
// block per GPU, the largest any layer allows (B <= 32, d_model * weight size
// <= 16 KiB, so d_model <= 8192).  Device code never names it: its address on
// each device comes from hipGetSymbolAddress, taken once per device with that
// device current.
constexpr size_t kStaticWorkFloats = (size_t)kMaxBatch * 8192;
static __device__ __align__(256) float scratch[kStaticWorkFloats];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static float *g_scratch_ptr[kMaxDevices];   // per device, null until first use

// The current device's copy of `scratch`, or null when its address cannot be
// taken.
static float *static_work() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = (float *)ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace asf

using namespace asf;

extern "C" {

#ifdef ASF_DEBUG
const char *asf_version(void) { return "asf 0.2 (gfx950, debug checks)"; }
#else
const char *asf_version(void) { return "asf 0.2 (gfx950)"; }
#endif

const char *asf_status_string(asf_status s) {
    switch (s) {
    case ASF_OK: return "ok";
    case ASF_ERR_ARG: return "invalid argument";
    case ASF_ERR_SHAPE: return "unsupported shape";
    case ASF_ERR_ALIGN: return "misaligned pointer or row length";
    case ASF_ERR_STORAGE: return "storage too small";
    case ASF_ERR_UNSUPPORTED: return "unsupported combination";
    case ASF_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

size_t asf_layer_storage_bytes(const asf_layer_desc *desc) {
    if (!desc || !desc_ok(*desc)) return 0;
    return carve(*desc, 0, nullptr) + 256;  // slack for aligning an unaligned base
}

asf_status asf_create_layer(const asf_layer_desc *desc, const asf_layer_weights *w,
                            const int32_t *neuron_table, void *storage, size_t storage_bytes,
                            void *stream, asf_layer **out) {
    if (out) *out = nullptr;
    if (!desc || !w || !storage || !out) return ASF_ERR_ARG;
    if (desc->d_model <= 0 || desc->d_ffn <= 0 || desc->pred_hidden <= 0 ||
        desc->max_batch <= 0 || (desc->gated != 0 && desc->gated != 1) ||
        (desc->wtype != ASF_F32 && desc->wtype != ASF_F16))
        return ASF_ERR_ARG;
    {
        const int ws = desc->wtype == ASF_F16 ? 2 : 4;
        if ((desc->d_model * ws) % (16 * kSlices) != 0 || (desc->pred_hidden * ws) % 16 != 0)
            return ASF_ERR_ALIGN;
    }
    if (!desc_ok(*desc)) return ASF_ERR_SHAPE;
    if (!w->w_up || !w->w_down || !w->p1 || !w->p2) return ASF_ERR_ARG;
    if (desc->gated ? !w->w_gate : w->w_gate != nullptr) return ASF_ERR_UNSUPPORTED;
    if (!aligned16(w->w_up) || !aligned16(w->w_down) || !aligned16(w->p1) || !aligned16(w->p2) ||
        (w->w_gate && !aligned16(w->w_gate)) || !aligned16(storage))
        return ASF_ERR_ALIGN;
    if (storage_bytes < asf_layer_storage_bytes(desc)) return ASF_ERR_STORAGE;

    asf_layer *L = new (std::nothrow) asf_layer;
    if (!L) return ASF_ERR_ARG;
    L->tracing = false;
    memset(&L->trace, 0, sizeof(L->trace));
    carve(*desc, (uintptr_t)storage, &L->v);
    LayerView &v = L->v;
    hipStream_t s = (hipStream_t)stream;
    const int ws = v.ws, d = v.d, f = v.f, H = v.H;
    hipError_t e = hipSuccess;
    auto chk = [&](hipError_t r) {
        if (e == hipSuccess && r != hipSuccess) e = r;
    };
    {
        int dev = 0;
        v.ncu = 0;
        chk(hipGetDevice(&dev));
        chk(hipDeviceGetAttribute(&v.ncu, hipDeviceAttributeMultiprocessorCount, dev));
        if (v.ncu < 1) v.ncu = 1;
    }
    // neuron table and its inverse
    if (neuron_table)
        chk(hipMemcpyAsync(v.perm, neuron_table, (size_t)f * 4, hipMemcpyDeviceToDevice, s));
    else
        chk(launch_invert(nullptr, f, v.perm, s));  // identity table
    chk(launch_invert(v.perm, f, v.inv, s));
    // predictor: layer 1 as given, layer 2 rows and bias in slot order
    chk(hipMemcpyAsync(v.p1, w->p1, (size_t)H * d * ws, hipMemcpyDeviceToDevice, s));
    chk(launch_gather_f32(w->c1, nullptr, H, v.c1, s));
    if (v.p2) {
        chk(hipMemsetAsync(v.p2, 0, (size_t)v.nq * kRowsPerWG * H * ws, s));
        chk(launch_perm_rows(w->p2, v.ch, v.perm, f, v.p2, v.ch, 0, v.nq, s));
    }
    chk(launch_p2_kmajor(w->p2, H, f, v.nq, ws, v.perm, v.p2k, s));
    chk(launch_gather_f32(w->c2, v.perm, f, v.c2, s));
    // neuron bundles: [gate,] up row, down column (W_down transposed), slot order
    const size_t bstride_chunks = (size_t)v.nmat * v.cd;
    const int up_idx = v.gated ? 1 : 0, dn_idx = v.nmat - 1;
    if (v.gated) chk(launch_perm_rows(w->w_gate, v.cd, v.perm, f, v.bundles, bstride_chunks, 0, 0, s));
    chk(launch_perm_rows(w->w_up, v.cd, v.perm, f, v.bundles, bstride_chunks,
                         (size_t)up_idx * v.cd, 0, s));
    chk(launch_transpose_perm(w->w_down, d, f, ws, v.inv, v.bundles, (size_t)v.nmat * d,
                              (size_t)dn_idx * d, s));
    chk(launch_gather_f32(w->b1, v.perm, f, v.b1, s));
    chk(launch_gather_f32(w->b2, nullptr, d, v.b2, s));
    chk(hipMemsetAsync(v.arrive, 0, kArrive * 4, s));
    // the batched FC1 reads x16's row padding (zero) against absent weights
    if (v.x16)
        chk(hipMemsetAsync(v.x16, 0, 2 * (size_t)v.max_batch * x16_pitch(v.d) * 2, s));
    // the one-launch step: exchange words tagged 0, epoch 1; used when every
    // owner can be resident at once
    chk(hipMemsetAsync(v.xch, 0, (size_t)kXchCopies * v.xstride * 8, s));
    chk(hipMemsetAsync(v.dbg, 0, 64, s));
    chk(hipMemsetD32Async((hipDeviceptr_t)v.epoch, 1, 1, s));
    v.fused = step1_fits(v) ? 1 : 0;
    if (e != hipSuccess) {
        delete L;
        return ASF_ERR_HIP;
    }
#ifdef ASF_DEBUG
    if (neuron_table) {
        // a permutation of 0 .. f-1: every entry in range, none repeated
        const asf_status st = debug_check_ids(v, neuron_table, nullptr, f, s);
        if (st != ASF_OK) {
            delete L;
            return st;
        }
    }
#endif
    *out = L;
    return ASF_OK;
}

void asf_destroy_layer(asf_layer *layer) { delete layer; }

static asf_status check_call(const asf_layer *layer, const float *x, int32_t B) {
    if (!layer || !x) return ASF_ERR_ARG;
    if (B < 1 || B > layer->v.max_batch) return ASF_ERR_SHAPE;
    if (!aligned16(x)) return ASF_ERR_ALIGN;
    return ASF_OK;
}

asf_status asf_predict(const asf_layer *layer, const float *x, int32_t B, int32_t *active,
                       int32_t *n_active, uint64_t *token_masks, void *stream) {
    asf_status st = check_call(layer, x, B);
    if (st != ASF_OK) return st;
    const LayerView &v = layer->v;
    hipStream_t s = (hipStream_t)stream;
    if (launch_pred_l1(v, x, B, layer->tr(), s) != hipSuccess) return ASF_ERR_HIP;
    if (launch_score(v, x, B, false, layer->tr(), s) != hipSuccess) return ASF_ERR_HIP;
    if ((active || n_active || token_masks) &&
        launch_list(v, B, active, n_active, token_masks, layer->tr(), s) != hipSuccess)
        return ASF_ERR_HIP;
    return ASF_OK;
}

asf_status asf_sparse_ffn(const asf_layer *layer, const float *x, int32_t B,
                          const int32_t *active, const int32_t *n_active, const float *residual,
                          float *y, void *stream) {
    asf_status st = check_call(layer, x, B);
    if (st != ASF_OK) return st;
    if (!y || (active && !n_active)) return ASF_ERR_ARG;
    if (!aligned16(y) || (residual && !aligned16(residual))) return ASF_ERR_ALIGN;
    const LayerView &v = layer->v;
    hipStream_t s = (hipStream_t)stream;
#ifdef ASF_DEBUG
    if (active) {
        const asf_status dst = debug_check_ids(v, active, n_active, 0, s);
        if (dst != ASF_OK) return dst;
    }
#endif
    if (B == 1) {
        // one token: the decode step's per-owner FC1 + FC2 over the last set
        // or the caller's list
        if (launch_ffn1(v, x, active, n_active, layer->tr(), s) != hipSuccess) return ASF_ERR_HIP;
        if (launch_fc2_sum(v, residual, y, layer->tr(), s) != hipSuccess) return ASF_ERR_HIP;
        return ASF_OK;
    }
    if (launch_fc1(v, x, B, active ? 1 : 0, active, n_active, layer->tr(), s) != hipSuccess)
        return ASF_ERR_HIP;
    if (launch_fc2(v, B, active != nullptr, residual, y, layer->tr(), s) != hipSuccess)
        return ASF_ERR_HIP;
    return ASF_OK;
}

int32_t asf_step_launches(const asf_layer *layer, int32_t B) {
    if (!layer || B < 1 || B > layer->v.max_batch) return 0;
    const LayerView &v = layer->v;
    if (B == 1) return v.fused ? 2 : 3;
    if (v.wtype != ASF_F16) return 4;
    // predictor layer 1 (with its slice sum from kPred1MaxB + 1 tokens on),
    // scores, FC1 (and its slice sum unless FC2 forms it), FC2 and its group
    // sum
    return (B <= kPred1MaxB ? 1 : 2) + 1 + (fc2_fuses_fin(v, B, false) ? 1 : 2) + 2;
}

asf_status asf_decode_step(const asf_layer *layer, const float *x, int32_t B,
                           const float *residual, float *y, int32_t *active, int32_t *n_active,
                           void *stream) {
    asf_status st = check_call(layer, x, B);
    if (st != ASF_OK) return st;
    if (!y) return ASF_ERR_ARG;
    if (!aligned16(y) || (residual && !aligned16(residual))) return ASF_ERR_ALIGN;
    const LayerView &v = layer->v;
    hipStream_t s = (hipStream_t)stream;
    if (launch_step(v, x, B, residual, y, active, n_active, layer->tr(), s) != hipSuccess)
        return ASF_ERR_HIP;
    return ASF_OK;
}

asf_status asf_exact_ffn(const asf_layer *layer, const float *x, int32_t B,
                         const float *residual, float *y, int32_t *active, int32_t *n_active,
                         void *stream) {
    asf_status st = check_call(layer, x, B);
    if (st != ASF_OK) return st;
    if (!y) return ASF_ERR_ARG;
    if (B != 1) return ASF_ERR_UNSUPPORTED;
    if (!aligned16(y) || (residual && !aligned16(residual))) return ASF_ERR_ALIGN;
    const LayerView &v = layer->v;
    hipStream_t s = (hipStream_t)stream;
    if (launch_exact1(v, x, false, layer->tr(), s) != hipSuccess) return ASF_ERR_HIP;
    if (launch_fc2_sum(v, residual, y, layer->tr(), s) != hipSuccess) return ASF_ERR_HIP;
    if ((active || n_active) &&
        launch_list(v, 1, active, n_active, nullptr, layer->tr(), s) != hipSuccess)
        return ASF_ERR_HIP;
    return ASF_OK;
}

asf_status asf_profile_activations(const asf_layer *layer, const float *x, int32_t n,
                                   uint32_t *counts, void *stream) {
    if (!layer || !x || !counts || n < 0) return ASF_ERR_ARG;
    if (!aligned16(x)) return ASF_ERR_ALIGN;
    const LayerView &v = layer->v;
    hipStream_t s = (hipStream_t)stream;
    for (int32_t t = 0; t < n; ++t) {
        if (launch_exact1(v, x + (size_t)t * v.d, true, nullptr, s) != hipSuccess)
            return ASF_ERR_HIP;
        if (launch_count_bits(v, counts, s) != hipSuccess) return ASF_ERR_HIP;
    }
    return ASF_OK;
}

asf_status asf_hot_first_table(const uint32_t *counts, int32_t d_ffn, int32_t *table,
                               void *stream) {
    if (!counts || !table || d_ffn <= 0 || d_ffn > kMaxFfn) return ASF_ERR_ARG;
    if (launch_rank_table(counts, d_ffn, table, (hipStream_t)stream) != hipSuccess)
        return ASF_ERR_HIP;
    return ASF_OK;
}

static asf_status check_stack(asf_layer *const *layers, int32_t n_layers, const float *x,
                              int32_t B, int32_t residual, const float *y, const float *work) {
    if (!layers || n_layers < 1 || !x || !y || (residual != 0 && residual != 1))
        return ASF_ERR_ARG;
    if (n_layers > 1 && !work) return ASF_ERR_ARG;
    if (!layers[0]) return ASF_ERR_ARG;
    const int d = layers[0]->v.d;
    for (int32_t l = 0; l < n_layers; ++l) {
        const asf_layer *L = layers[l];
        if (!L) return ASF_ERR_ARG;
        if (L->v.d != d) return ASF_ERR_SHAPE;
        if (B < 1 || B > L->v.max_batch) return ASF_ERR_SHAPE;
        for (int32_t m = 0; m < l; ++m)
            if (layers[m] == L) return ASF_ERR_ARG;
    }
    if (!aligned16(x) || !aligned16(y) || (work && !aligned16(work))) return ASF_ERR_ALIGN;
    if (n_layers > 1) {
        const uintptr_t bytes = (uintptr_t)B * d * 4;
        auto overlap = [&](const void *a, const void *b) {
            const uintptr_t p = (uintptr_t)a, q = (uintptr_t)b;
            return p < q + bytes && q < p + bytes;
        };
        if (overlap(work, x) || overlap(work, y)) return ASF_ERR_ARG;
    }
    return ASF_OK;
}

asf_status asf_stack_decode(asf_layer *const *layers, int32_t n_layers, const float *x,
                            int32_t B, int32_t residual, float *y, float *work, void *stream) {
    const asf_status st = check_stack(layers, n_layers, x, B, residual, y, work);
    if (st != ASF_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    // layer l writes y when (n_layers - 1 - l) is even, else work, so the
    // last layer lands in y; layer 0 reads x, every later layer its
    // predecessor's output
    const float *in = x;
    for (int32_t l = 0; l < n_layers; ++l) {
        const LayerView &v = layers[l]->v;
        const asf::Trace *tr = layers[l]->tr();
        float *out = ((n_layers - 1 - l) % 2 == 0) ? y : work;
        if (launch_step(v, in, B, residual ? in : nullptr, out, nullptr, nullptr, tr, s) !=
            hipSuccess)
            return ASF_ERR_HIP;
        in = out;
    }
    return ASF_OK;
}

asf_status asf_stack_decode_static(asf_layer *const *layers, int32_t n_layers, const float *x,
                                   int32_t B, int32_t residual, float *y, void *stream) {
    if (!layers || n_layers < 1 || !layers[0]) return ASF_ERR_ARG;
    if (B < 1 || (size_t)B * (size_t)layers[0]->v.d > kStaticWorkFloats) return ASF_ERR_SHAPE;
    float *work = nullptr;
    if (n_layers > 1) {
        work = static_work();
        if (!work) return ASF_ERR_HIP;
    }
    return asf_stack_decode(layers, n_layers, x, B, residual, y, work, stream);
}

asf_status asf_stack_decode_lookahead(asf_layer *const *layers, int32_t n_layers,
                                      const float *x, int32_t residual, float *y, float *work,
                                      void *stream) {
    const asf_status st = check_stack(layers, n_layers, x, 1, residual, y, work);
    if (st != ASF_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    // layer 0's set from its own input
    {
        const LayerView &v = layers[0]->v;
        if (launch_pred_l1(v, x, 1, layers[0]->tr(), s) != hipSuccess ||
            launch_score(v, x, 1, false, layers[0]->tr(), s) != hipSuccess)
            return ASF_ERR_HIP;
    }
    // layer l: its FC1/FC2 rows beside layer l+1's predictor layer 1 (both
    // on layer l's input), then layer l+1's scores beside layer l's output
    const float *in = x;
    for (int32_t l = 0; l < n_layers; ++l) {
        const LayerView &v = layers[l]->v;
        const LayerView *vn = l + 1 < n_layers ? &layers[l + 1]->v : nullptr;
        float *out = ((n_layers - 1 - l) % 2 == 0) ? y : work;
        if (launch_ffn1_pred1(v, vn, in, layers[l]->tr(), s) != hipSuccess ||
            launch_score1_fc2sum(vn, v, residual ? in : nullptr, out, layers[l]->tr(), s) !=
                hipSuccess)
            return ASF_ERR_HIP;
        in = out;
    }
    return ASF_OK;
}

asf_status asf_dense_ffn_ref(const asf_layer *layer, const float *x, int32_t B,
                             const float *residual, float *y, void *stream) {
    asf_status st = check_call(layer, x, B);
    if (st != ASF_OK) return st;
    if (!y) return ASF_ERR_ARG;
    if (!aligned16(y) || (residual && !aligned16(residual))) return ASF_ERR_ALIGN;
    const LayerView &v = layer->v;
    hipStream_t s = (hipStream_t)stream;
    if (launch_fc1(v, x, B, 2, nullptr, nullptr, layer->tr(), s) != hipSuccess)
        return ASF_ERR_HIP;
    if (launch_fc2(v, B, false, residual, y, layer->tr(), s, true) != hipSuccess)
        return ASF_ERR_HIP;
    return ASF_OK;
}

size_t asf_head_predictor_storage_bytes(const asf_head_desc *desc) {
    if (!desc || !head_desc_ok(*desc)) return 0;
    return carve_heads(*desc, 0, nullptr) + 256;
}

asf_status asf_create_head_predictor(const asf_head_desc *desc, const asf_head_weights *w,
                                     void *storage, size_t storage_bytes, void *stream,
                                     asf_head_predictor **out) {
    if (out) *out = nullptr;
    if (!desc || !w || !storage || !out || !w->q1 || !w->q2) return ASF_ERR_ARG;
    if (desc->wtype != ASF_F32 && desc->wtype != ASF_F16) return ASF_ERR_ARG;
    if (!head_desc_ok(*desc)) return ASF_ERR_SHAPE;
    if (!aligned16(w->q1) || !aligned16(w->q2) || !aligned16(storage)) return ASF_ERR_ALIGN;
    if (storage_bytes < asf_head_predictor_storage_bytes(desc)) return ASF_ERR_STORAGE;
    asf_head_predictor *P = new (std::nothrow) asf_head_predictor;
    if (!P) return ASF_ERR_ARG;
    carve_heads(*desc, (uintptr_t)storage, &P->v);
    {
        int dev = 0;
        P->v.ncu = 1;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&P->v.ncu, hipDeviceAttributeMultiprocessorCount, dev) !=
                hipSuccess || P->v.ncu < 1)
            P->v.ncu = 1;
    }
    const HeadView &v = P->v;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipSuccess;
    auto chk = [&](hipError_t r) {
        if (e == hipSuccess && r != hipSuccess) e = r;
    };
    chk(hipMemcpyAsync(v.q1, w->q1, (size_t)v.H * v.d * v.ws, hipMemcpyDeviceToDevice, s));
    chk(launch_gather_f32(w->c1, nullptr, v.H, v.c1, s));
    chk(hipMemcpyAsync(v.q2, w->q2, (size_t)v.nh * v.H * v.ws, hipMemcpyDeviceToDevice, s));
    chk(launch_gather_f32(w->c2, nullptr, v.nh, v.c2, s));
    if (e != hipSuccess) {
        delete P;
        return ASF_ERR_HIP;
    }
    *out = P;
    return ASF_OK;
}

void asf_destroy_head_predictor(asf_head_predictor *hp) { delete hp; }

asf_status asf_predict_heads(const asf_head_predictor *hp, const float *x, int32_t B,
                             uint64_t *head_masks, int32_t *heads, int32_t *n_sel,
                             void *stream) {
    if (!hp || !x || (!head_masks && !heads && !n_sel)) return ASF_ERR_ARG;
    if (B < 1 || B > hp->v.max_batch) return ASF_ERR_SHAPE;
    if (!aligned16(x)) return ASF_ERR_ALIGN;
    if (launch_head_predict(hp->v, x, B, head_masks, heads, n_sel, (hipStream_t)stream) !=
        hipSuccess)
        return ASF_ERR_HIP;
    return ASF_OK;
}

asf_status asf_layer_set_trace(asf_layer *layer, void *const *events, int32_t n) {
    if (!layer || n < 0 || n > ASF_K_COUNT) return ASF_ERR_ARG;
    memset(&layer->trace, 0, sizeof(layer->trace));
    layer->tracing = events != nullptr && n > 0;
    if (layer->tracing)
        for (int i = 0; i < 2 * n; ++i) layer->trace.ev[i] = (hipEvent_t)events[i];
    return ASF_OK;
}

}  // extern "C"
