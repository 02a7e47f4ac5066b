/*
 * fq.h -- C ABI of libfq: 4-bit weight + 4-bit KV-cache decoding of OPT-style
 * decoder layers on one AMD MI355X (gfx950).
 *
 * The method is FlexGen's (Sheng et al., "High-Throughput Generative Inference
 * of Large Language Models with a Single GPU"): weights and the attention KV
 * cache are compressed to 4 bits (FlexGen README, key features, "Extreme
 * Compression"; pith.science abstract), compute runs on the reconstructed
 * values, weights that do not fit in device memory are streamed layer by
 * layer from pinned host memory with copies overlapped with compute (README,
 * "Benchmark Results" discussion of the block schedule; awesome-repositories
 * feature "Asynchronous Tensor Loading"), and throughput is generated tokens
 * divided by prompt time plus generation time (README, "Benchmark Results",
 * Metric bullet).
 *
 * Readings this library fixes where the pages are silent (the pages state only
 * "4 bits"):
 *   - group = 64 consecutive elements along the contiguous (last) axis;
 *   - asymmetric min/max: code = clamp(rint_half_even((x - min) / s), 0, 15),
 *     s = fp16((max - min) / 15) computed in IEEE fp32; min and s stored as an
 *     fp16 pair per group; a -0 minimum and a zero scale are stored as +0;
 *   - nibble order: element 2k in the low nibble of byte k;
 *   - reconstruction for GEMM operands: fp16(min + code * s), one rounding.
 *
 * Conventions for every call:
 *   - fp16 values travel as uint16_t bit patterns.
 *   - Pointers documented "device" are HIP device memory owned by the caller;
 *     "host" pointers are host memory owned by the caller.  No call keeps a
 *     caller pointer after it returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls are asynchronous on that stream unless stated otherwise.
 *   - Every call returns an fq_status; on failure fq_last_error() gives a
 *     thread-local message.  Nothing aborts and no C++ exception crosses the
 *     ABI.  Shape errors are detected on the host before any launch.
 *   - Handles are not thread-safe; distinct handles may be used concurrently.
 */
#ifndef FQ_H
#define FQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FQ_OK = 0,
  FQ_ERR_INVALID = -1,     /* bad argument or shape */
  FQ_ERR_UNSUPPORTED = -2, /* valid request outside what this library implements */
  FQ_ERR_OOM = -3,         /* device or pinned-host allocation failed */
  FQ_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed */
} fq_status;

#define FQ_GROUP 64

/* Thread-local text of the last non-OK status ("" if none). */
const char* fq_last_error(void);
/* Library version string. */
const char* fq_version(void);

/* ------------------------------------------------------------------------ */
/* Packed 4-bit tensor.  Logical fp16 matrix [rows, cols], cols % 64 == 0.
 *   codes: device uint8  [rows, cols/2]        row-major, nibble pairs
 *   meta:  device uint16 [rows, cols/64, 2]    fp16 {min, scale} per group   */
typedef struct {
  uint8_t* codes;
  uint16_t* meta;
  int64_t rows;
  int64_t cols;
  int32_t group; /* must be 64 */
} fq_packed;

/* Quantise an fp16 matrix group-wise to 4 bits (FlexGen README, "Extreme
 * Compression": weights and attention cache stored in 4 bits).
 *   x:   device fp16 [rows, cols], row stride ldx elements (ldx >= cols)
 *   out: codes/meta device buffers of the sizes above; out->rows/cols must
 *        equal rows/cols and out->group must be 64.
 * Bit-exact with the reading in the header comment.  Errors: FQ_ERR_INVALID
 * for cols % 64 != 0, ldx < cols, null pointers; FQ_ERR_UNSUPPORTED for a
 * group other than 64. */
fq_status fq_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, const fq_packed* out,
                      void* stream);

/* Reconstruct a packed matrix to fp16: y[r, c] = fp16(min + code * s).
 *   y: device fp16 [rows, cols] contiguous.  (Debug and test helper.) */
fq_status fq_dequantize(const fq_packed* in, uint16_t* y, void* stream);

/* ------------------------------------------------------------------------ */
/* Weight operand of a projection: W [N = out features, K = in features],
 * either 4-bit packed (groups along K) or plain fp16 row-major [N, K]. */
typedef enum { FQ_WEIGHT_PACKED4 = 0, FQ_WEIGHT_F16 = 1 } fq_weight_kind;

typedef struct {
  int32_t kind;        /* fq_weight_kind */
  fq_packed packed;    /* kind == FQ_WEIGHT_PACKED4: rows = N, cols = K */
  const uint16_t* w16; /* kind == FQ_WEIGHT_F16: device fp16 [N, K] */
  int64_t n;           /* N */
  int64_t k;           /* K, multiple of 64 */
} fq_weight;

/* Epilogue flags of fq_dequant_gemm, applied in this order in fp32:
 *   BIAS:     v += bias[n]
 *   QSCALE:   v *= qscale for columns n < qscale_cols (query scaling d^-1/2)
 *   RELU:     v = max(v, 0)
 *   RESIDUAL: v += residual[m, n]
 * then one rounding to fp16 (or an fp32 store with F32OUT). */
enum {
  FQ_EPI_BIAS = 1u << 0,
  FQ_EPI_QSCALE = 1u << 1,
  FQ_EPI_RELU = 1u << 2,
  FQ_EPI_RESIDUAL = 1u << 3,
  FQ_EPI_F32OUT = 1u << 4
};

/* C[M, N] = epilogue(A[M, K] * W^T) with the weight reconstructed in
 * registers (fp16) and fp32 accumulation on the matrix cores: the
 * dequant-fused projection GEMM of the QKV, output and FFN layers.  The pages
 * store the weights in 4 bits and compute on them (FlexGen README, "Extreme
 * Compression", and its --compress-weight flag under "Handle Out-of-memory";
 * the Manning "FlexGen technique" page, "Configuring an OPT model": weight
 * compression is a policy switch); the projections of an OPT layer are the
 * models the README benchmarks ("Benchmark Results": OPT-6.7B/30B/175B).
 * Fusing the reconstruction into the product is this library's design.
 *   A:        device fp16, row stride lda (>= K)
 *   bias:     device fp16 [N] (FQ_EPI_BIAS) or NULL
 *   residual: device fp16, row stride ldr (FQ_EPI_RESIDUAL) or NULL; may alias C
 *             only when ldr == ldc (each element is read before it is written)
 *   C:        device fp16 (or fp32 with FQ_EPI_F32OUT), row stride ldc (>= N)
 * M may be 0 (no-op).  Errors: FQ_ERR_INVALID for K % 64 != 0, strides too
 * small, null pointers required by the flags. */
fq_status fq_dequant_gemm(const uint16_t* A, int64_t M, int64_t lda, const fq_weight* W, const uint16_t* bias,
                          const uint16_t* residual, int64_t ldr, uint32_t epilogue, float qscale,
                          int64_t qscale_cols, void* C, int64_t ldc, void* stream);

/* fq_dequant_gemm for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments, kernels and results (bit for bit), but the fp32
 * split-K partials of the small-M kernels go to a fixed 64 MiB scratch
 * array that the library holds in each GPU's memory from its load until the
 * process ends, instead of a workspace grown with hipMalloc.  The call
 * allocates nothing and records no fq_timing_* events.
 *   Errors: those of fq_dequant_gemm, and FQ_ERR_INVALID when a shape would
 *   need more than 64 MiB of partials (the message gives the size; at batch
 *   144 the four OPT-175B decode products need at most 61 MiB, the QKV
 *   product's three slabs of 144 x 36864; at batch 256 that product needs
 *   72 MiB and is rejected).
 * Calls that overlap on one GPU (several streams or host threads) share that
 * GPU's scratch and race; serialise them.  Nothing in the scratch needs to
 * start at zero (every partial read is written first in the same call). */
fq_status fq_dequant_gemm_noalloc(const uint16_t* A, int64_t M, int64_t lda, const fq_weight* W,
                                  const uint16_t* bias, const uint16_t* residual, int64_t ldr, uint32_t epilogue,
                                  float qscale, int64_t qscale_cols, void* C, int64_t ldc, void* stream);

/* ------------------------------------------------------------------------ */
/* One layer of KV cache (device memory; caller- or handle-owned).
 * 4-bit cache (bits 4, or 0 in a zero-initialised struct):
 *   k_codes, v_codes: uint8  [batch, heads, capacity, head_dim/2]
 *   k_meta,  v_meta:  uint16 [batch, heads, capacity, head_dim/64, 2]
 * One group = 64 consecutive head-dim channels of one token and head, so a
 * group never spans two tokens.  head_dim % 64 == 0.
 * fp16 cache (bits 16; cache compression switched off while weights may still
 * be compressed -- FlexGen README, "Handle Out-of-memory", where weight
 * compression is a flag of its own, and the Manning "FlexGen technique" page,
 * "Configuring an OPT model", where the policy sets weight and cache
 * compression separately):
 *   k16, v16: fp16 [batch, heads, capacity, head_dim]; the codes/meta
 *   pointers are unused. */
typedef struct {
  uint8_t* k_codes;
  uint16_t* k_meta;
  uint8_t* v_codes;
  uint16_t* v_meta;
  int64_t batch;
  int32_t heads;
  int32_t head_dim;
  int64_t capacity;
  int32_t group; /* must be 64 */
  int32_t bits;  /* 4 (or 0): packed codes + meta;  16: fp16 entries in k16 / v16 */
  uint16_t* k16;
  uint16_t* v16;
} fq_kv_layer;

/* Quantise-on-append: the new tokens' K and V (fp16) become 4-bit cache
 * entries (FlexGen README, "Extreme Compression": the attention cache is
 * stored in 4 bits); with bits == 16 they are copied unchanged.
 *   k, v: device fp16; row r = b*T + t holds heads*head_dim values of token
 *         t of sequence b; row stride ld elements (e.g. the K and V column
 *         blocks of a fused QKV activation with ld = 3*hidden)
 *   writes cache positions pos..pos+T-1 of sequences b0..b0+B-1.
 * Errors: FQ_ERR_INVALID if b0+B > batch or pos+T > capacity. */
fq_status fq_kv_append(const fq_kv_layer* kv, const uint16_t* k, const uint16_t* v, int64_t ld, int64_t b0,
                       int64_t B, int64_t T, int64_t pos, void* stream);

/* Decode attention over the cache: for each sequence b and head h,
 * s_j = q . k^_j for j < len, p = softmax(s), o = sum_j p_j v^_j, with k^, v^
 * reconstructed in registers in fp32 (min + code * s) from a 4-bit cache, or
 * read as stored from an fp16 cache.  The attention cache is the one the
 * pages compress to 4 bits (FlexGen README, "Extreme Compression"; the
 * paper's abstract on the pith.science record: weights and the attention
 * cache compressed to 4 bits); one decode step is one generated token of the
 * README's "Benchmark Results" workload (output length 32).  Scores and the
 * softmax are fp32; the value pass multiplies each position's probability by
 * its group scale and a power of two (2^-E, 2^E just above the largest such
 * scale the lane has seen) and rounds that product to fp16 before the fp32
 * dot product with the exact codes; the group minima enter in fp32.  Error of
 * that rounding per output element: at most 2^-11 * sum_j p_j s_j |c_j| /
 * sum_j p_j, plus 2^-25 * 2^E * 15 per term below fp16's normal range.
 *   q:   device fp16 [B, heads*head_dim] row stride ldq, already scaled by
 *        head_dim^-1/2
 *   out: device fp16 [B, heads*head_dim] row stride ldo
 *   uses cache sequences b0..b0+B-1, positions 0..len-1 (1 <= len <= capacity).
 * Errors: FQ_ERR_INVALID if b0+B > batch, len outside [1, capacity] or above
 * 30000 (the scores are held in LDS), strides below heads*head_dim or ldq
 * not a multiple of 8, or q/out NULL or q not 16-byte aligned;
 * FQ_ERR_UNSUPPORTED for a group other than 64 or head_dim other than 64/128. */
fq_status fq_decode_attention(const uint16_t* q, int64_t ldq, const fq_kv_layer* kv, int64_t b0, int64_t B,
                              int64_t len, uint16_t* out, int64_t ldo, void* stream);

/* Causal attention of T new tokens at positions pos..pos+T-1 (already
 * appended to the cache): query t sees cache positions 0..pos+t -- the
 * prompt pass of the README's "Benchmark Results" workload (input length 512)
 * over the 4-bit attention cache ("Extreme Compression").  On the matrix
 * cores with the codes as exact fp16 integers: per quantisation group g the
 * scores are s_g (q . c) + min_g sum(q_g), in log2 units, in fp32 (the min
 * terms as a product of the fp16 minima with each group sum split into two
 * fp16 parts, 22 significant bits); the values take the codes
 * centred (c - 8) against fp16(p * s_g * 2^-E_g) (2^E_g just above the
 * largest value scale of the group among the keys read), the minima (+ 8 s)
 * in fp32.  An fp16 cache is read as stored.
 *   q: device fp16 rows b*T + t, stride ldq (scaled);  out: same layout, ldo.
 * Errors: FQ_ERR_INVALID if b0+B > batch, pos+T > capacity, strides below
 * heads*head_dim or not multiples of 8, or q/out NULL or not 16-byte aligned. */
fq_status fq_prefill_attention(const uint16_t* q, int64_t ldq, const fq_kv_layer* kv, int64_t b0, int64_t B,
                               int64_t T, int64_t pos, uint16_t* out, int64_t ldo, void* stream);

/* QKV projection with the K/V append fused into its epilogue (FlexGen
 * README, "Extreme Compression": the attention cache is stored in 4 bits; the
 * fusion is this library's): the same results as
 *   fq_dequant_gemm(A, M, lda, W, bias, NULL, 0, BIAS | QSCALE, qscale, h, C, ldc)
 *   fq_kv_append(kv, C + h, C + 2h, ldc, b0, B, T, pos)
 * bit for bit (q columns of C, cache codes and {min, scale} or fp16 entries).
 *   W: [3h, K] rows q | k | v with h = kv->heads * kv->head_dim;  bias [3h] or NULL
 *   A: device fp16 [M, K], M = B * T, row b*T + t = token t of sequence b0 + b
 *   C: device fp16 [M, >= 3h] (ldc); columns [0, h) receive the scaled queries.
 *      Columns [h, 3h) are written only where the fused form does not apply
 *      (small M, fp16 weights, misaligned buffers); callers read only q.
 * Errors: FQ_ERR_INVALID for M != B*T, W->n != 3h, ranges beyond the cache,
 * and the argument errors of the two calls above. */
fq_status fq_qkv_gemm_append(const uint16_t* A, int64_t M, int64_t lda, const fq_weight* W, const uint16_t* bias,
                             float qscale, const fq_kv_layer* kv, int64_t b0, int64_t B, int64_t T, int64_t pos,
                             uint16_t* C, int64_t ldc, void* stream);

/* LayerNorm over rows: y = (x - mean) / sqrt(var + eps) * gamma + beta with
 * fp32 statistics (biased variance) and one rounding to fp16.
 *   x, y: device fp16 [M, h] with strides ldx, ldy;  gamma, beta: device fp16 [h]. */
fq_status fq_layernorm(const uint16_t* x, int64_t M, int64_t h, int64_t ldx, const uint16_t* gamma,
                       const uint16_t* beta, float eps, uint16_t* y, int64_t ldy, void* stream);

/* ------------------------------------------------------------------------ */
/* Model description (OPT-style pre-LayerNorm decoder, ReLU FFN). */
typedef struct {
  int32_t hidden;  /* h */
  int32_t heads;   /* H, head_dim = h / H (multiple of 64) */
  int32_t ffn;     /* F */
  int32_t layers;  /* L */
  int32_t vocab;   /* V (0: no embedding / LM head; layer-only model) */
  int32_t max_pos; /* rows of the learned position table (positions used: p + 2) */
} fq_model_config;

/* Placement policy (FlexGen README, "Get Started": --percent places weights
 * and cache; "Handle Out-of-memory": --compress-weight, --pin-weight). */
typedef struct {
  int32_t compress_weight; /* 1: 4-bit packed weights (group 64); 0: fp16 weights */
  int32_t compress_cache;  /* 1: 4-bit KV cache (group 64); 0: fp16 KV cache */
  int32_t resident_layers; /* layers 0..resident_layers-1 are kept in HBM; the rest live in
                              pinned host memory -- packed (0.5625 byte per weight) when
                              compress_weight, else fp16 -- and are streamed through two
                              device staging buffers; -1 = all resident */
  int32_t host_layers;     /* streamed layers: distinct host layer blobs; layer l reads blob
                              (l - resident_layers) % host_layers; 0 = one per layer */
  int32_t overlap;         /* 1: prefetch layer l+1 on a copy stream while layer l computes */
  int64_t max_tokens;      /* rows of the per-call activation workspace (0: default 16384) */
  int32_t cache_resident_layers; /* KV cache placement (README, "Get Started": the --percent pair
                              for the cache): layers 0..n-1 keep their cache in HBM, the rest in
                              pinned host memory, staged through two device buffers per pass
                              (the valid prefix copied in, the new positions copied back);
                              -1 = all in HBM */
} fq_policy;

typedef struct fq_model fq_model;
typedef struct fq_kv fq_kv;

/* fp16 parameters of one layer (device pointers; the library copies or
 * quantises them, it does not keep the pointers). */
typedef struct {
  const uint16_t* w_qkv; /* [3h, h] rows: q features, then k, then v */
  const uint16_t* w_out; /* [h, h] */
  const uint16_t* w_fc1; /* [F, h] */
  const uint16_t* w_fc2; /* [h, F] */
  const uint16_t* b_qkv; /* [3h] */
  const uint16_t* b_out; /* [h] */
  const uint16_t* b_fc1; /* [F] */
  const uint16_t* b_fc2; /* [h] */
  const uint16_t* ln1_g;
  const uint16_t* ln1_b;
  const uint16_t* ln2_g;
  const uint16_t* ln2_b;
} fq_layer_weights;

/* Create a model handle: device storage for every resident layer (packed
 * 4-bit weights when the policy compresses them: 0.5625 byte per weight, the
 * README's "around 70%" saving of --compress-weight under "Handle
 * Out-of-memory"; else fp16), pinned host blobs for the streamed layers and
 * their two device staging buffers (README, "Get Started": --percent places
 * weights on the GPU or the CPU; the block schedule of "Benchmark Results"
 * overlaps their copies with compute), and the activation workspace.  The
 * parameters are uninitialised until fq_model_set_layer /
 * fq_model_init_random.  The handle owns every allocation.  Errors:
 * FQ_ERR_INVALID for bad sizes, FQ_ERR_UNSUPPORTED for a head_dim other
 * than 64 or 128, FQ_ERR_OOM when device or pinned memory runs out (nothing
 * is leaked). */
fq_status fq_model_create(const fq_model_config* cfg, const fq_policy* policy, fq_model** out);
/* Free everything the handle owns (waits for the device first).  NULL is a no-op. */
fq_status fq_model_destroy(fq_model* m);

/* Quantise (or copy) one layer's fp16 parameters into the model's store:
 * the load-time weight compression of the README's --compress-weight
 * ("Handle Out-of-memory"; "Extreme Compression"), group-wise as fq_quantize.
 * A streamed layer is packed on the device and copied to its pinned host blob
 * (synchronous on `stream`); its staged copies are forgotten so that the next
 * pass copies the new weights in.  Errors: FQ_ERR_INVALID for a layer out of
 * range or a NULL parameter. */
fq_status fq_model_set_layer(fq_model* m, int32_t layer, const fq_layer_weights* w, void* stream);

/* Token embedding [V, h], position table [max_pos, h], final LN gamma/beta [h]
 * (device fp16; copied).  The LM head is tied to the token embedding, and
 * position p reads row p + 2 of the position table (the OPT models of the
 * README's "Benchmark Results").  FQ_ERR_INVALID for a layer-only model
 * (vocab 0). */
fq_status fq_model_set_embeddings(fq_model* m, const uint16_t* embed, const uint16_t* pos,
                                  const uint16_t* lnf_g, const uint16_t* lnf_b, void* stream);

/* Random initialisation of every parameter on the device from the
 * counter-based generator SplitMix64 (Steele, Lea, Flood 2014):
 * element i of stream s is mix64(key(seed, s) + (i+1) * 0x9E3779B97F4A7C15);
 * its four 16-bit lanes are summed (Irwin-Hall, centred) and scaled in fp32
 * to std sigma, then rounded to fp16.  Weights: sigma 0.02.  bias_sigma == 0:
 * biases 0, LN gamma 1, beta 0; otherwise biases/betas sigma bias_sigma and
 * gammas sigma 1.  Linear weights are then quantised (compress_weight) or
 * stored fp16 (resident or in pinned host memory).  Synchronous. */
fq_status fq_model_init_random(fq_model* m, uint64_t seed, double bias_sigma, void* stream);

/* Device view of one layer's packed weight (which: 0 qkv, 1 out, 2 fc1, 3 fc2),
 * owned by the model.  FQ_ERR_INVALID if weights are not compressed or the
 * layer is streamed from host memory. */
fq_status fq_model_packed_weight(const fq_model* m, int32_t layer, int32_t which, fq_packed* out);

/* Parity-test hook: record what one layer computes inside later calls
 * (fq_layer_step, fq_generate), so that a test can feed the oracle the same
 * inputs and the same fp16 K/V -- its quantisation of those K/V must then
 * equal the cache bit for bit, and the layer's outputs are compared under
 * teacher forcing.  Not part of the method; off unless set.
 *   layer:   the layer whose values are recorded
 *   b0, nb:  sequences b0..b0+nb-1
 *   capacity: positions per sequence in each buffer
 *   x_in, y_out, k16, v16, x1: device fp16 [nb, capacity, hidden] or NULL;
 *     row (b - b0, p) receives the layer's input row, its output row, the
 *     fp16 K and V it appends, and its residual after the output projection,
 *     at position p of sequence b.
 * While a capture is set for a layer, that layer's QKV projection runs as the
 * two calls fq_qkv_gemm_append is defined to equal (projection, then
 * append), so K and V exist in fp16.  The buffers must stay valid while the
 * capture is set.  fq_model_set_capture(m, NULL, 0) clears every capture.
 * Errors: FQ_ERR_INVALID for more than 8 captures, two on one layer, a layer
 * out of range; a later call fails with FQ_ERR_INVALID if it reaches a
 * position at or beyond `capacity` of a captured sequence. */
typedef struct {
  int32_t layer;
  int64_t b0;
  int64_t nb;
  int64_t capacity;
  uint16_t* x_in;
  uint16_t* y_out;
  uint16_t* k16;
  uint16_t* v16;
  uint16_t* x1; /* the residual after the output projection, x + o Wo^T + bo */
} fq_capture;
fq_status fq_model_set_capture(fq_model* m, const fq_capture* caps, int32_t n);

/* KV cache for `batch` sequences of up to `capacity` positions, all layers:
 * 4-bit (0.5625 byte per cached element) when the policy compresses the
 * cache, else fp16 (2 bytes) -- the attention cache the pages compress to 4
 * bits (FlexGen README, "Extreme Compression").  Layers at or beyond the
 * policy's cache_resident_layers live in pinned host memory (README, "Get
 * Started": the --percent pair for the cache places it on the GPU or the
 * CPU); fq_kv_layer_view then returns host pointers.  The handle owns every
 * allocation.  Errors: FQ_ERR_INVALID for bad sizes, FQ_ERR_OOM when memory
 * runs out (nothing is leaked). */
fq_status fq_kv_create(const fq_model* m, int64_t batch, int64_t capacity, fq_kv** out);
/* Free everything the handle owns (waits for the device first).  NULL is a no-op. */
fq_status fq_kv_destroy(fq_kv* kv);
/* The buffers of one layer's cache (device pointers, or pinned host pointers
 * for an offloaded layer), owned by the handle. */
fq_status fq_kv_layer_view(const fq_kv* kv, int32_t layer, fq_kv_layer* out);

/* One decoder layer over T new tokens of sequences b0..b0+B-1 at positions
 * pos..pos+T-1: LN1, QKV projection (+bias, query scaling), quantise-on-
 * append of K/V (or fp16 append), attention over the cache (causal for T > 1), output
 * projection (+bias, +residual), LN2, FC1 (+bias, ReLU), FC2 (+bias,
 * +residual).  The layer is that of the OPT models the pages run (FlexGen
 * README, "Get Started with a Single GPU" and "Benchmark Results":
 * OPT-6.7B/30B/175B), pre-LayerNorm with a ReLU FFN, its weights and
 * attention cache in 4 bits ("Extreme Compression").  T > 1 is the prompt
 * pass, T == 1 one generation step; both count in the README's throughput
 * ("Benchmark Results", Metric bullet).
 * Each of these values is rounded once to fp16 (round to nearest even) from
 * its fp32 accumulation, and nowhere else:
 *   h1 = LN1(x);  q = (h1 Wq^T + bq) * head_dim^-1/2;  k = h1 Wk^T + bk;
 *   v = h1 Wv^T + bv  (k, v then quantised into the cache, or kept fp16);
 *   o = attention(q, cache);  x1 = x + o Wo^T + bo;  h2 = LN2(x1);
 *   f = max(h2 W1^T + b1, 0);  y = x1 + f W2^T + b2.
 * LayerNorm: eps 1e-5, biased variance, fp32 statistics.
 *   x, y: device fp16 [B*T, h] (may be the same buffer).
 * B*T must not exceed the policy's max_tokens.  Layers whose fp16 weights
 * live in host memory are copied in synchronously on `stream` first.
 * Errors: FQ_ERR_INVALID for a layer out of range, B*T above max_tokens,
 * sequences or positions beyond the cache, NULL or misaligned x/y. */
fq_status fq_layer_step(fq_model* m, int32_t layer, fq_kv* kv, int64_t b0, int64_t B, int64_t T, int64_t pos,
                        const uint16_t* x, uint16_t* y, void* stream);

/* Generation statistics (README, "Benchmark Results", Metric bullet:
 * throughput = generated tokens / (prompt time + generation time)). */
typedef struct {
  double prefill_s;      /* prompt processing, incl. the first generated token */
  double decode_s;       /* the remaining gen_len-1 steps */
  double tokens_per_s;   /* B * gen_len / (prefill_s + decode_s) */
  double h2d_bytes;      /* weight bytes streamed from host memory */
  double h2d_s;          /* weight copy-stream busy time (sum of copy intervals) */
  double kv_h2d_bytes;   /* cache bytes staged in from host memory (offloaded layers) */
  double kv_d2h_bytes;   /* cache bytes written back to host memory */
} fq_gen_stats;

/* Greedy generation: embed the prompt, prefill every layer (prompt chunked
 * by sequences to fit max_tokens), final LN, LM head (tied embedding, fp32
 * logits), argmax (ties to the lowest id) gives token 1; then gen_len-1
 * decode steps.
 *   prompt_ids: host int32 [B, P];  out_ids: host int32 [B, gen_len]
 *   kv: a cache with batch >= B and capacity >= P + gen_len - 1
 *   logits: optional device fp32 [gen_len, B, V] (NULL to skip)
 * Synchronous: returns after the last token is on the host.  Timing uses
 * HIP events on `stream`. */
fq_status fq_generate(fq_model* m, fq_kv* kv, const int32_t* prompt_ids, int64_t B, int64_t P, int64_t gen_len,
                      int32_t* out_ids, float* logits, fq_gen_stats* stats, void* stream);

/* Optional progress report for long generations: fq_generate calls
 * fn(done, gen_len, user) once per generated token, in order
 * (done = 1..gen_len), from the calling thread, after that token's step has
 * finished on the device -- while it queues later steps (a non-blocking
 * query between steps) and, once everything is queued, by waiting for the
 * remaining steps in order.  NULL disables it (the default).  Process-wide;
 * not synchronised with concurrent fq_generate calls.  The device timing is
 * unchanged. */
typedef void (*fq_progress_fn)(int64_t done, int64_t total, void* user);
void fq_set_progress(fq_progress_fn fn, void* user);

/* ------------------------------------------------------------------------ */
/* Per-launch device timing (HIP events on the launching stream), grouped by
 * kernel class, with each launch's algorithmic work: flops of the
 * contraction and the bytes a single pass over its operands moves to or
 * from HBM (packed weights 0.5625 B/element, fp16 2 B, fp32 4 B).  Used by
 * the benchmark to report each kernel against its roofline (FlexGen README,
 * "Benchmark Results": the pages report only end-to-end throughput; the
 * per-kernel split is this library's). */
typedef enum {
  FQ_KC_GEMM_PREFILL = 0, /* projection GEMMs with M > 256 rows */
  FQ_KC_GEMM_DECODE = 1,  /* projection GEMMs with M <= 256 rows */
  FQ_KC_LM_HEAD = 2,      /* fp32-output GEMMs (LM head) */
  FQ_KC_DECODE_ATTN = 3,
  FQ_KC_PREFILL_ATTN = 4,
  FQ_KC_KV_APPEND = 5,
  FQ_KC_QUANTIZE = 6,
  FQ_KC_LAYERNORM = 7,
  FQ_KC_COUNT = 8
} fq_kernel_class;

#define FQ_KC_ALL 0xFFu

typedef struct {
  int64_t launches;
  double seconds; /* sum of per-launch device time */
  double flops;   /* sum of algorithmic flops */
  double bytes;   /* sum of algorithmic HBM bytes */
  int64_t dropped; /* launches of this class not timed: the event pool
                      (65536 launches per recording) was exhausted */
} fq_kernel_stats;

/* Start recording the launches of the classes whose bit (1u << class) is set
 * in class_mask (FQ_KC_ALL: every class); clears earlier records.  Launches
 * of other classes record nothing.  Process-wide.  The event pool holds at
 * most 65536 launches per recording; later launches are counted in
 * `dropped` and not timed. */
fq_status fq_timing_start(uint32_t class_mask);
/* Stop, wait for the recorded events and fill out[FQ_KC_COUNT] (may be NULL).
 * FQ_ERR_HIP if an event cannot be read. */
fq_status fq_timing_stop(fq_kernel_stats* out);

/* ------------------------------------------------------------------------ */
/* Seeded synthetic inputs (the generator described at fq_model_init_random):
 * fill device fp16 dst[0..n) with elements first..first+n-1 of stream `stream_id`. */
fq_status fq_synth_normal_f16(uint16_t* dst, int64_t n, uint64_t seed, uint64_t stream_id, int64_t first,
                              double sigma, void* stream);
/* Token ids ((u >> 32) * vocab) >> 32 into device int32 dst[0..n). */
fq_status fq_synth_token_ids(int32_t* dst, int64_t n, uint64_t seed, uint64_t stream_id, int32_t vocab,
                             void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FQ_H */
