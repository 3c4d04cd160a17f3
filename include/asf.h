/*
 * asf.h -- C ABI of the activation-sparse FFN decode library (libasf.so),
 * hand-written HIP for gfx950 (MI355X).
 *
 * The calls follow the problem statement of the pages:
 *   1. load a layer's weights and its predictor, arranged through a neuron
 *      table that maps each stored neuron to its original position
 *      ("LLM模型之PowerInfer1.0" §4.2; "PowerInfer: Nhanh Large Language Model
 *      với GPU Tiêu dùng", section "Đặt vị trí và Quản lý Nơ-ron");
 *   2. predict which neurons the current input activates with a two-layer
 *      X-H-O MLP ("LLM模型之PowerInfer1.0" §1 and appendix "DejaVu");
 *   3. compute only those neurons: FC1 as a dot product with each active
 *      neuron row, FC2 as an AXPY over the matching contiguous columns of the
 *      down projection ("LLM模型之PowerInfer1.0" §2.1 Fig. 1, §4.4 and "其他"
 *      question 3);
 *   4. the dense FFN over all neurons as the comparison ("Técnicas dispersas
 *      para una aceleración 100X…", section "Viabilidad de la sparsidad de
 *      activación").
 *
 * Memory and ownership
 *   - Every tensor argument is a DEVICE pointer allocated by the caller; the
 *     library allocates no device memory.  The only host-side allocation is
 *     the small opaque asf_layer handle.
 *   - asf_create_layer copies the weights into caller-provided `storage`
 *     (size from asf_layer_storage_bytes) in the library's own layout; the
 *     original weight buffers may be freed once the copy has run on `stream`.
 *     `storage` must outlive the handle.  Per-call scratch (predictor hidden
 *     vector, masks, active list, partial sums) also lives in `storage`, so a
 *     layer serves one call at a time: calls on one layer must be ordered
 *     (same stream, or synchronised).
 *   - All calls are asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL means the default stream).  No call synchronises the device, and
 *     the active count never travels to the host.
 *
 * Data types
 *   Weights (FFN matrices and predictor matrices) are all ASF_F32 or all
 *   ASF_F16 (IEEE binary16 bits).  Biases, x, h, y are float32.  Products are
 *   accumulated in float32.
 *
 * Errors
 *   Every call validates its arguments on the host and returns a status
 *   without touching the device when they are invalid.  Launch failures are
 *   reported as ASF_ERR_HIP.  Device-side faults surface at the caller's next
 *   synchronisation.  No C++ exception crosses this ABI.  Neuron ids in a
 *   caller-supplied active list that are out of range are skipped; duplicate
 *   ids are the caller's error (one token counts such a neuron once, a batch
 *   as often as it is listed).
 *
 * Debug build
 *   libasf_debug.so (the same kernels, the host API compiled with ASF_DEBUG)
 *   checks the device content the release library takes on trust, and synchronises
 *   the stream to do so: asf_sparse_ffn returns ASF_ERR_ARG for a caller
 *   list with an id out of range or listed twice, or a count outside
 *   0 .. d_ffn; asf_create_layer for a neuron table that is not a
 *   permutation of 0 .. d_ffn-1.  asf_version names the library variant.
 */
#ifndef ASF_H
#define ASF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct asf_layer asf_layer; /* opaque host handle */

typedef enum { ASF_F32 = 0, ASF_F16 = 1 } asf_dtype;

typedef enum {
    ASF_OK = 0,
    ASF_ERR_ARG = 1,         /* null pointer or invalid scalar argument */
    ASF_ERR_SHAPE = 2,       /* dimension out of the supported range */
    ASF_ERR_ALIGN = 3,       /* pointer or row length not 16-byte aligned */
    ASF_ERR_STORAGE = 4,     /* storage smaller than asf_layer_storage_bytes */
    ASF_ERR_UNSUPPORTED = 5, /* valid but unsupported combination */
    ASF_ERR_HIP = 6          /* a HIP runtime call or kernel launch failed */
} asf_status;

/* Shape and numeric options of one FFN layer.
 *   d_model      input/output width d (rows of W_down, columns of W_up)
 *   d_ffn        number of FFN neurons f (1 .. 65536)
 *   pred_hidden  hidden size H of the X-H-O predictor
 *   max_batch    largest B any call will use (1 .. 32)
 *   gated        0: a_i = ReLU(W_up[i].x + b1_i)
 *                1: a_i = ReLU(W_gate[i].x + b1_i) * (W_up[i].x)
 *                   (ReLU in place of SiLU on the gate; the gate decides the
 *                   true active set)
 *   wtype        asf_dtype of every weight matrix
 *   threshold    logit threshold theta: neuron i is predicted active when
 *                its score s_i > theta (strict).  0 is the sigmoid-0.5
 *                decision of the pages' per-output binary classifier.
 * Alignment: d_model * sizeof(weight) must be a multiple of 256 bytes
 * (d_model % 128 == 0 for ASF_F16, % 64 for ASF_F32; the FC2 kernel splits
 * d_model into 16 slices of whole 16-byte chunks) and pred_hidden *
 * sizeof(weight) a multiple of 16 bytes.  Limits: d_model * sizeof(weight)
 * <= 16 KiB, pred_hidden * sizeof(weight) <= 4 KiB. */
typedef struct {
    int32_t d_model;
    int32_t d_ffn;
    int32_t pred_hidden;
    int32_t max_batch;
    int32_t gated;
    int32_t wtype;
    float threshold;
} asf_layer_desc;

/* Original weights, DEVICE pointers, row-major in nn.Linear layouts:
 *   w_up, w_gate [d_ffn][d_model]  (w_gate only when gated, else NULL)
 *   b1           [d_ffn] float32 or NULL (= 0); the gate bias when gated
 *   w_down       [d_model][d_ffn]
 *   b2           [d_model] float32 or NULL (= 0)
 *   p1           [pred_hidden][d_model]     predictor layer 1
 *   c1           [pred_hidden] float32 or NULL (= 0)
 *   p2           [d_ffn][pred_hidden]       predictor layer 2
 *   c2           [d_ffn] float32 or NULL (= 0)
 * Matrices must be 16-byte aligned. */
typedef struct {
    const void *w_up;
    const void *w_gate;
    const float *b1;
    const void *w_down;
    const float *b2;
    const void *p1;
    const float *c1;
    const void *p2;
    const float *c2;
} asf_layer_weights;

/* Bytes of device storage a layer with this descriptor needs (weights in the
 * library layout plus per-call scratch).  Returns 0 for an invalid desc. */
size_t asf_layer_storage_bytes(const asf_layer_desc *desc);

/* Copy a layer into `storage` in hot-first, neuron-major layout and return a
 * handle.
 *   neuron_table  DEVICE int32 [d_ffn]: neuron_table[slot] = original id of
 *                 the neuron stored at `slot` (a permutation of 0..d_ffn-1;
 *                 hot neurons first).  NULL = identity.  It is not checked
 *                 on the device: a table that is not a permutation leaves
 *                 the layer's content undefined (never out-of-bounds).
 *   storage       DEVICE, 256-byte aligned, >= asf_layer_storage_bytes.
 * The layout work runs asynchronously on `stream`; the handle is usable by
 * later work on the same stream at once.  *out receives the handle, or NULL
 * on error. */
asf_status asf_create_layer(const asf_layer_desc *desc, const asf_layer_weights *w,
                            const int32_t *neuron_table, void *storage,
                            size_t storage_bytes, void *stream, asf_layer **out);

/* Free the host handle (never the caller's storage).  NULL is a no-op. */
void asf_destroy_layer(asf_layer *layer);

/* Predict the active neurons of B tokens (X-H-O predictor, then threshold,
 * then compaction of the union of the tokens' sets).
 *   x            DEVICE float32 [B][d_model]
 *   B            1 .. max_batch
 *   active       DEVICE int32 [d_ffn] or NULL: receives the ORIGINAL ids of
 *                the union of the B tokens' active sets, in ascending stored
 *                (slot) order; entries past *n_active are left untouched
 *   n_active     DEVICE int32 [1] or NULL: receives the count
 *   token_masks  DEVICE uint64 [B][ceil(d_ffn/64)] or NULL: per-token
 *                bitmasks in STORED (slot) order, bit (slot % 64) of word
 *                (slot / 64)
 * The union list is also kept in the layer's scratch, where asf_sparse_ffn
 * with active == NULL reads it. */
asf_status asf_predict(const asf_layer *layer, const float *x, int32_t B,
                       int32_t *active, int32_t *n_active, uint64_t *token_masks,
                       void *stream);

/* FFN over a neuron set: y[b] = residual[b] + b2 + sum_{i in S} a_{b,i} W_down[:, i]
 * with a_{b,i} the FC1 (gated) activation of neuron i for token b.
 *   x         DEVICE float32 [B][d_model]
 *   active    DEVICE int32 original ids (distinct, any order), or NULL to use
 *             the layer's last set (of asf_predict, asf_decode_step or
 *             asf_exact_ffn)
 *   n_active  DEVICE int32 [1] count of `active` (ignored when active == NULL;
 *             required otherwise)
 *   residual  DEVICE float32 [B][d_model] or NULL (= 0)
 *   y         DEVICE float32 [B][d_model]; may alias residual
 * For B > 1 every token computes every neuron of the set (the union of the
 * batch's sets when the set comes from asf_predict).  One token runs the
 * decode step's own FC1 + FC2 kernels (each owner workgroup takes the ids
 * whose stored slot it owns), so asf_predict followed by this call, with
 * active == NULL or with the predicted list, gives asf_decode_step's y bit
 * for bit. */
asf_status asf_sparse_ffn(const asf_layer *layer, const float *x, int32_t B,
                          const int32_t *active, const int32_t *n_active,
                          const float *residual, float *y, void *stream);

/* One decode step of one layer: asf_predict followed by asf_sparse_ffn over
 * the predicted union set, with no host round trip in between.  The optional
 * outputs are those of asf_predict.  One token: two kernels when every
 * owner workgroup can be resident at once (predictor layers 1 and 2,
 * threshold, FC1 and each owner's FC2 into one row; the sum of the owner
 * rows), else three (predictor layer 1 as a kernel of its own); both forms
 * give the same bits (asf_step_launches tells which runs).  The results are
 * bit-identical to asf_predict followed by asf_sparse_ffn with active ==
 * NULL, and repeated calls give identical bits. */
asf_status asf_decode_step(const asf_layer *layer, const float *x, int32_t B,
                           const float *residual, float *y, int32_t *active,
                           int32_t *n_active, void *stream);

/* One decode step of B tokens through a stack of layers, in order:
 *   x_0 = x;  x_{l+1} = FFN_l(x_l) + (residual ? x_l : 0);  y = x_n
 * where FFN_l is layer l's decode step (asf_decode_step: predictor, threshold,
 * FC1 and FC2 over the predicted set).  The pages give every layer its own
 * predictor, sized by that layer's skew ("LLM模型之PowerInfer1.0" §4.1), and
 * run the layers one after another.
 *   layers    HOST array of n_layers >= 1 handles, all with the same d_model
 *             and max_batch >= B; a handle may appear once only (each layer's
 *             scratch serves one step at a time)
 *   x         DEVICE float32 [B][d_model], read only unless y == x
 *   residual  0: x_{l+1} = FFN_l(x_l);  1: x_{l+1} = x_l + FFN_l(x_l)
 *   y         DEVICE float32 [B][d_model]; may equal x
 *   work      DEVICE float32 [B][d_model] scratch, overlapping neither x nor y
 *             (may be NULL when n_layers == 1)
 * Asynchronous on `stream`; launches the decode step's kernels per layer. */
asf_status asf_stack_decode(asf_layer *const *layers, int32_t n_layers, const float *x,
                            int32_t B, int32_t residual, float *y, float *work, void *stream);

/* asf_stack_decode without a caller work buffer, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The [B][d_model] float32 buffer between
 * layers is the library's own static device array of 32 * 8192 floats
 * (1 MiB per GPU, held until the process ends), which covers every shape a
 * layer accepts (B <= 32, d_model <= 8192); a larger B * d_model returns
 * ASF_ERR_SHAPE.  The call allocates nothing.  Every call on one GPU shares
 * that GPU's array: calls that overlap on one GPU (other streams, other
 * threads) race and must be ordered by the caller.  The first call on a
 * device takes the array's address there (hipGetSymbolAddress); failure
 * returns ASF_ERR_HIP.  Arguments and results otherwise as asf_stack_decode
 * with work == NULL (y == x allowed). */
asf_status asf_stack_decode_static(asf_layer *const *layers, int32_t n_layers, const float *x,
                                   int32_t B, int32_t residual, float *y, void *stream);

/* asf_stack_decode for one token with the look-ahead predictor (the
 * asynchronous reading of DejaVu, "LLM模型之PowerInfer1.0" appendix "DejaVu",
 * Eq. -2): layer l+1's set is predicted from layer l's INPUT, so its
 * predictor runs beside layer l's FC1/FC2:
 *   S_0 = predict_0(x_0);  S_l = predict_l(x_{l-1}) for l >= 1;
 *   x_{l+1} = FFN_l(x_l over S_l) + (residual ? x_l : 0);  y = x_n
 * Arguments as asf_stack_decode with B = 1.  Two launches per layer on
 * `stream`: layer l's FC1/FC2 owner rows together with layer l+1's
 * predictor layer 1, then layer l+1's scores together with layer l's
 * output (layers of another weight type than their predecessor get their
 * predictor layer 1 as a launch of its own).  Per layer the results equal
 * asf_predict on x_{l-1} followed by asf_sparse_ffn (active == NULL) on
 * x_l, bit for bit. */
asf_status asf_stack_decode_lookahead(asf_layer *const *layers, int32_t n_layers,
                                      const float *x, int32_t residual, float *y, float *work,
                                      void *stream);

/* Dense comparator: the same FFN over all d_ffn neurons. */
asf_status asf_dense_ffn_ref(const asf_layer *layer, const float *x, int32_t B,
                             const float *residual, float *y, void *stream);

/* Exact-mask FFN of one token, without the predictor: every neuron's
 * pre-activation z_i = W_up[i] . x + b1_i (W_gate when gated) is computed,
 * the set is the true one, {i : z_i > 0}, and FC2 reads only that set's down
 * columns (the gated form also only its up rows):
 *   y = residual + b2 + sum_{z_i > 0} a_i W_down[:, i]
 * which equals the dense FFN (ReLU(z) is 0 off the set) up to the order of
 * the fp32 additions.  The pages rest the method on this exact zero pattern
 * of the ReLU ("Técnicas dispersas para una aceleración 100X…", section
 * "Viabilidad de la sparsidad de activación"); it reads all of W_up (W_gate)
 * and the active fraction of W_down.
 *   x, residual, y   as asf_sparse_ffn, with B == 1 (ASF_ERR_UNSUPPORTED
 *                    otherwise)
 *   active, n_active DEVICE int32 [d_ffn] / [1], or NULL: the true set as
 *                    original ids in ascending stored (slot) order, as
 *                    asf_predict gives its set
 * Kernels: FC1 (pre-activations, mask, gated up rows, owner FC2 rows), FC2
 * (sum of the owner rows), then LIST when an output is requested. */
asf_status asf_exact_ffn(const asf_layer *layer, const float *x, int32_t B,
                         const float *residual, float *y, int32_t *active, int32_t *n_active,
                         void *stream);

/* Activation profiler, the offline half of the neuron table: for each of the
 * n tokens of x, every neuron's true pre-activation is computed (as in
 * asf_exact_ffn) and counts[id] is incremented for the neurons with z > 0,
 * indexed by ORIGINAL id ("LLM模型之PowerInfer1.0" §5.1: the activation
 * frequency of each neuron over a general dataset).  The layer's own table
 * only fixes the storage order; create it with table == NULL to profile.
 *   x       DEVICE float32 [n][d_model], n >= 0
 *   counts  DEVICE uint32 [d_ffn], accumulated (the caller zeroes it first)
 * Uses the layer's scratch like every other call; two small kernels per
 * token, asynchronous on `stream`. */
asf_status asf_profile_activations(const asf_layer *layer, const float *x, int32_t n,
                                   uint32_t *counts, void *stream);

/* Hot-first neuron table from activation counts: table[s] = the original id
 * with the s-th largest count, ties broken by the smaller id -- the neuron
 * impact of "LLM模型之PowerInfer1.0" §5.2 Eq. 1 (impact = activation
 * frequency) in descending order, the layout asf_create_layer takes.
 *   counts  DEVICE uint32 [d_ffn];  table  DEVICE int32 [d_ffn]
 * d_ffn in 1 .. 65536.  One kernel (exact ranking), asynchronous. */
asf_status asf_hot_first_table(const uint32_t *counts, int32_t d_ffn, int32_t *table,
                               void *stream);

/* ---------------------------------------------------------------------------
 * Attention-head predictor ("LLM模型之PowerInfer1.0", appendix "DejaVu",
 * the SP_A model of Eq. -1): per transformer layer a second two-layer MLP
 * whose output layer has one unit per attention head, each a sigmoid
 * select / skip decision, so only the selected heads need to run.  Here the
 * decision is taken on the logit: head j is selected when
 *   s_j = Q2[j] . ReLU(Q1 x + c1) + c2_j  >  threshold   (strict; 0 is the
 *   sigmoid-0.5 decision).
 * Run on layer l's input y_l it gives layer l's heads (Eq. -1); run on y_l
 * with layer l+1's weights it is the look-ahead form of Eq. -2 (the same call
 * on another input).  Attention itself and the KV cache are not part of
 * this library.
 * ------------------------------------------------------------------------- */
typedef struct asf_head_predictor asf_head_predictor; /* opaque host handle */

/* Shape of one head predictor:
 *   d_model      input width d
 *   n_heads      outputs, one per attention head (1 .. 4096)
 *   pred_hidden  hidden size H
 *   max_batch    largest B any call will use (1 .. 32)
 *   wtype        asf_dtype of Q1 and Q2
 *   threshold    logit threshold theta
 * Alignment and limits as asf_layer_desc: d_model * sizeof(weight) a
 * multiple of 256 bytes, at most 16 KiB; pred_hidden * sizeof(weight) a
 * multiple of 16 bytes, at most 4 KiB. */
typedef struct {
    int32_t d_model;
    int32_t n_heads;
    int32_t pred_hidden;
    int32_t max_batch;
    int32_t wtype;
    float threshold;
} asf_head_desc;

/* DEVICE pointers, row-major: q1 [pred_hidden][d_model], c1 [pred_hidden]
 * float32 or NULL (= 0), q2 [n_heads][pred_hidden], c2 [n_heads] float32 or
 * NULL (= 0).  Matrices 16-byte aligned. */
typedef struct {
    const void *q1;
    const float *c1;
    const void *q2;
    const float *c2;
} asf_head_weights;

/* Device storage bytes of a head predictor (weights + per-call scratch);
 * 0 for an invalid desc. */
size_t asf_head_predictor_storage_bytes(const asf_head_desc *desc);

/* Copy the weights into caller storage (DEVICE, 256-byte aligned, at least
 * asf_head_predictor_storage_bytes) on `stream` and return a handle in *out
 * (NULL on error).  The originals may be freed once the copy has run. */
asf_status asf_create_head_predictor(const asf_head_desc *desc, const asf_head_weights *w,
                                     void *storage, size_t storage_bytes, void *stream,
                                     asf_head_predictor **out);

/* Free the host handle (never the caller's storage).  NULL is a no-op. */
void asf_destroy_head_predictor(asf_head_predictor *hp);

/* Selected heads of B tokens, each token on its own (no union):
 *   x           DEVICE float32 [B][d_model]
 *   head_masks  DEVICE uint64 [B][ceil(n_heads/64)] or NULL: bit (j % 64) of
 *               word (j / 64) set when head j is selected
 *   heads       DEVICE int32 [B][n_heads] or NULL: token b's selected heads
 *               in ascending order at heads[b][0 .. n_sel[b]); the rest of
 *               the row is left untouched
 *   n_sel       DEVICE int32 [B] or NULL: the count per token
 * At least one output must be given (ASF_ERR_ARG otherwise).  Two kernels
 * (layer 1; layer 2 + threshold + masks), a third for the lists when
 * n_heads > 64.  The handle's scratch serves one call at a time. */
asf_status asf_predict_heads(const asf_head_predictor *hp, const float *x, int32_t B,
                             uint64_t *head_masks, int32_t *heads, int32_t *n_sel, void *stream);

/* Kernels behind the calls (ids for asf_layer_set_trace).
 *   asf_predict       PRED_L1, SCORE, then LIST when an output is requested
 *   asf_decode_step   PRED_L1, SCORE_FC1 (B == 1; else SCORE + FC1), FC2,
 *                     then LIST when an output is requested (for one token
 *                     the list runs in FC2's grid, timed as FC2); one token
 *                     on a layer whose owners fit the device at once: SCORE_FC1
 *                     (with predictor layer 1), FC2 (asf_step_launches);
 *                     B >= 2 with fp16 weights: a phase can be two launches,
 *                     its events spanning both
 *   asf_sparse_ffn    FC1, FC2
 *   asf_dense_ffn_ref FC1 (every neuron), FC2
 *   asf_exact_ffn     FC1 (pre-activations, true set, owner FC2 rows), FC2
 *                     (sum of the owner rows), then LIST when requested */
typedef enum {
    ASF_K_PRED_L1 = 0,   /* predictor layer 1 GEMV */
    ASF_K_SCORE = 1,     /* predictor layer 2 GEMV + threshold -> mask bits */
    ASF_K_SCORE_FC1 = 2, /* the same, then FC1 of the predicted neurons; for one
                            token also their FC2 into one row per owner */
    ASF_K_FC1 = 3,       /* FC1 (+ReLU) of a neuron set */
    ASF_K_FC2 = 4,       /* FC2 column gather + reduction -> y; for one token in a
                            decode step, the sum of the owner rows -> y */
    ASF_K_LIST = 5,      /* slot-ordered masks and active list */
    ASF_K_COUNT = 6
} asf_kernel_id;

/* Kernel tracing, for measuring each kernel with HIP events on the stream it
 * runs on.  `events` holds 2*n hipEvent_t handles (as void*), n <= ASF_K_COUNT:
 * every later call on this layer launches kernel k with events[2k] as its
 * start and events[2k+1] as its stop event (hipExtLaunchKernelGGL: the
 * dispatch itself takes the events, so their difference is the kernel's own
 * duration); NULL entries are skipped.  events == NULL or n == 0 turns
 * tracing off.  The handles are borrowed: the caller creates and destroys
 * them. */
asf_status asf_layer_set_trace(asf_layer *layer, void *const *events, int32_t n);

/* Kernel launches of one asf_decode_step of `layer` for B tokens, a list
 * kernel of a batch left out.  One token: 2 when the step runs predict, FC1
 * and the owner FC2 rows in one launch (SCORE_FC1: the owners compute
 * predictor layer 1 and exchange h through device memory, which needs every
 * owner workgroup resident at once; the layer checks this at creation)
 * followed by the owner-row sum (FC2), else 3 (PRED_L1, SCORE_FC1, FC2).
 * B >= 2 traces four phases, PRED_L1, SCORE, FC1 and FC2: with fp32 weights
 * one launch each (4); with fp16 weights FC2 is two launches (the stream
 * kernel and its sum of group partials), FC1 too (its sum of k-slice
 * partials) except on plain layers with d_model <= 5120 at B <= 4, where the
 * FC2 stream kernel forms the activations itself, and predictor layer 1 is
 * two from 5 tokens on (5 to 7 in all), a phase's events spanning its
 * launches.  A caller tracing kernels learns from it which ids a step
 * uses.  0 for a null layer or B outside 1 .. max_batch. */
int32_t asf_step_launches(const asf_layer *layer, int32_t B);

/* Human-readable name of a status code (static string). */
const char *asf_status_string(asf_status s);

/* Library version string. */
const char *asf_version(void);

#ifdef __cplusplus
}
#endif
#endif /* ASF_H */
