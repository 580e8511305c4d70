/*
 * fa.h - FlashAttention for AMD Instinct MI355X (gfx950), C ABI: the forward
 * pass (bf16 and FP8), a split-KV forward for decode and small batches, and
 * the bf16 backward pass.
 *
 * The library computes exact scaled-dot-product attention
 *     O = softmax(scale * Q K^T) V,   LSE_i = log sum_j exp(scale * q_i . k_j)
 * without ever materialising the N x N score matrix: Q, K and V are tiled
 * through on-chip memory and the softmax is taken online, with a running row
 * maximum and row sum and a rescaling of the output accumulator (droidorbit
 * FlashAttention-3 explainer, "Mathematical Formulation: The Online Softmax
 * Rescaling Trick"; dibro.site FlashAttention-3 post, "Arquitectura y
 * metodo"). Causal attention skips key tiles that lie wholly after every
 * query of a query tile (dibro.site post, "Contribuciones clave").
 *
 * Conventions shared by every entry point
 *   - Tensors are contiguous row-major [B, H, N, d]: element (b, h, n, i) is
 *     at offset ((b*H + h)*N + n)*d + i. Q, K, V and O share one N
 *     (self-attention lengths) and one d.
 *   - bf16 tensors hold the bit patterns of bfloat16 (torch.bfloat16).
 *     fp8 tensors hold OCP e4m3fn bytes (torch.float8_e4m3fn).
 *   - LSE is float32 [B, H, N], the natural log of sum_j exp(scale*q_i.k_j)
 *     over the keys row i attends. It may be NULL to skip its store.
 *   - Causal (causal != 0): query i attends key j only when j <= i.
 *   - All tensor pointers are DEVICE pointers owned by the caller, 16-byte
 *     aligned. The library never frees or keeps them. Outputs must not
 *     overlap the inputs or each other: the kernels read inputs while other
 *     workgroups write outputs (not checked here; the Python binding checks).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream)
 *     of the calling thread's current device, which also holds the tensors.
 *     Calls only enqueue work and return; the caller keeps buffers alive
 *     until the stream has completed them. Faults inside a kernel surface at
 *     the caller's next synchronisation, not in the return code.
 *   - Arguments are validated on the host before any HIP call, in the order
 *     listed for each function. No C++ exception crosses this boundary.
 *     Nothing is printed unless the environment variable FA_LOG=1 is set.
 *   - Thread-safe and re-entrant. The state the library keeps: one memory
 *     pool per device for stream-ordered scratch (entry points that need
 *     scratch say so), created on first use under a lock, its memory
 *     allocated and freed in stream order (hipMallocFromPoolAsync /
 *     hipFreeAsync on `stream`) and retained for reuse until the process
 *     ends instead of being released after every call; and the fixed scratch
 *     array of the allocation-free entry point (fa_fwd_splitkv_noalloc),
 *     which is shared by its calls on a device.
 *   - Debugging aid: the environment variable FA_DEBUG (read at every call;
 *     bit 0 runs the forward and backward kernels' workgroups in reverse
 *     order, bit 1 fills the forward kernels' on-chip tile memory with NaN
 *     bytes before any tile is copied in) leaves every result bit for bit
 *     unchanged; it exists to show exactly that.
 */
#ifndef FA_H
#define FA_H

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_dtype {
    FA_BF16 = 0,      /* bf16 Q/K/V in, bf16 O out                                */
    FA_FP8_E4M3 = 1   /* bf16 Q/K/V in, quantised to e4m3 inside the call, bf16 O  */
} fa_dtype;

typedef enum fa_status {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = -1,   /* null pointer, non-positive size, bad scale     */
    FA_ERR_UNSUPPORTED = -2,   /* head dimension or dtype not instantiated       */
    FA_ERR_MISALIGNED = -3,    /* a tensor pointer is not 16-byte aligned        */
    FA_ERR_HIP = -4,           /* the HIP runtime reported an error at launch    */
    FA_ERR_TOO_LARGE = -5,     /* N*d above 2^30, B*H above the 32-bit range, or
                                  a launch grid above 2^32 - 1 work-items     */
    FA_ERR_SCRATCH_LIMIT = -6  /* the call needs more scratch than the
                                  allocation-free entry point holds           */
} fa_status;

/* Rows per FP8 quantisation block: one fp32 scale per 128 consecutive
 * sequence rows of one (batch, head), all d columns. */
#define FA_FP8_BLOCK 128

/*
 * fa_fwd - attention forward pass.
 *
 * q, k, v : bf16 [B, H, N, d] (inputs)       o : bf16 [B, H, N, d] (output)
 * lse     : float32 [B, H, N] or NULL         scale : softmax scale, finite > 0
 *           (callers normally pass 1/sqrt(d), the equation's scaling)
 * d       : 64, 96, 128 or 256 for FA_BF16; 64, 128 or 256 for FA_FP8_E4M3
 * dtype   : FA_BF16 runs the bf16 matrix-core path. With few query tiles
 *           in all (B*H*ceil(N/128) <= 128, causal <= 224), N >= 4096,
 *           N*d <= 2^29, d in {64, 96, 128} and an automatic split count
 *           (fa_splitkv_splits) of at least 2, it runs the split-KV path of
 *           fa_fwd_splitkv instead (stream-ordered scratch from the
 *           library's pool): the same products and softmax over key ranges,
 *           partial results merged by LSE, so the output differs from the
 *           one-pass kernel's only by rounding order.
 *           FA_FP8_E4M3 runs the FP8 path end to end on bf16 inputs: Q and K
 *           are rotated by a fixed random-sign Hadamard matrix and all three
 *           are block-quantised to e4m3, then the fa_fwd_fp8 kernel runs.
 *           K and V are quantised in one launch (fa_quant_fp8's arithmetic)
 *           into stream-ordered scratch (the library's pool, on `stream`);
 *           each workgroup of the forward kernel quantises its own 128-row
 *           Q block with the same arithmetic, so the output equals
 *           fa_quant_fp8 + fa_fwd_fp8 bit for bit. The fixed signs: sign i is -1 where the top bit of
 *           SplitMix64(0x5A17C0DE + i) is set, else +1 (SplitMix64: Steele,
 *           Lea, Flood 2014; the state is incremented by the golden gamma
 *           before mixing). d must be a power of two.
 * Validation order: null q/k/v/o -> INVALID_ARG; B, H or N < 1 -> INVALID_ARG;
 * dtype unknown or d unsupported -> UNSUPPORTED; scale not finite and > 0 ->
 * INVALID_ARG; N*d > 2^30, B*H >= 2^31 or B*H*ceil(N/128) >= 2^24 (one
 * 256-thread workgroup per 128 rows; a dispatch counts at most 2^32 - 1
 * work-items) -> TOO_LARGE; a pointer not 16-byte aligned -> MISALIGNED;
 * launch (or scratch allocation) error -> HIP.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, int causal, float scale, int dtype,
           void* stream);

/*
 * fa_quant_fp8 - block quantisation of one bf16 tensor to e4m3fn
 * (QbitAI FlashAttention-3 article, FP8 section: block-wise quantisation and
 * incoherent processing; FlashAttention-3 (HE), FP8 with reduced
 * quantisation error: rotation by a random orthogonal Hadamard matrix).
 *
 * x      : bf16 [B, H, N, d] (input)       x8 : e4m3fn [B, H, N, d] (output)
 * scales : float32 [B, H, ceil(N/128)] (output): dequantised value of an
 *          element = e4m3 value * scales[b, h, n/128].
 * per_tensor : 0 = one scale per 128-row block; 1 = one scale for the whole
 *          tensor, written to every entry of `scales`.
 * signs  : NULL (no rotation) or float32 [d] of +-1 on the device: x is
 *          rotated to x diag(signs) H_d / sqrt(d), H_d the Sylvester Hadamard
 *          matrix (d a power of two). Rotate Q and K with the same signs,
 *          never V.
 * Quantisation: y = x diag(signs) H_d (y = x without rotation), s = amax|y|
 * / 448 over the block (1 for an all-zero block), code = the e4m3 value
 * nearest to y / s (ties to even, clamped to +-448); the stored scale is s,
 * or s / sqrt(d) with rotation. The kernel takes y, s and the scaled value
 * in float32 and applies the scale as a product with its correctly rounded
 * reciprocal, so a code can differ from that of the exact y / s only where
 * y / s lies within a few float32 ulps of the midpoint between two e4m3
 * values (then it is the other of the two).
 * Validation order: null x/x8/scales -> INVALID_ARG; B, H or N < 1 ->
 * INVALID_ARG; d not in {64, 96, 128, 256}, or signs given and d not a power
 * of two -> UNSUPPORTED; the size limits of fa_fwd -> TOO_LARGE; misaligned -> MISALIGNED;
 * launch error -> HIP.
 */
int fa_quant_fp8(const void* x, void* x8, float* scales,
                 int B, int H, int N, int d, int per_tensor, const float* signs,
                 void* stream);

/*
 * fa_fwd_fp8 - attention forward pass on e4m3 operands with float32
 * accumulation and an fp32 online softmax (QbitAI article, FP8 section;
 * vikram-blog FlashAttention-3 post, "Production Gotchas": softmax state
 * stays in FP32).
 *
 * q8, k8, v8 : e4m3fn [B, H, N, d] with block scales q_scale, k_scale,
 *              v_scale : float32 [B, H, ceil(N/128)] as fa_quant_fp8 writes
 *              (positive; a non-positive V scale yields finite but
 *              meaningless rows).
 * o : bf16 [B, H, N, d]; lse : float32 [B, H, N] or NULL; d : 64, 128, 256.
 * The probabilities P of a key tile are multiplied by 64 * r and rounded
 * to e4m3 for the P V product, r = (V scale of the tile's block) / (a
 * reference V scale): the reference starts at the largest V block scale of
 * the (b, h) and moves to a tile's own scale whenever r would leave
 * [2^-4, 1] (the float32 accumulator is then rescaled). With V block
 * scales of any spread, all-zero blocks included, 64 * r * P >= 4 * P,
 * so every P >= 2^-8 (relative to the row's reference maximum) stays in
 * e4m3's normal range. The row sum is the float32
 * accumulation of those same rounded values divided by r (taken on the
 * matrix cores), so O is normalised by the weights it was formed with.
 * Validation order as fa_fwd (null scale arrays -> INVALID_ARG).
 */
int fa_fwd_fp8(const void* q8, const void* k8, const void* v8,
               const float* q_scale, const float* k_scale, const float* v_scale,
               void* o, float* lse, int B, int H, int N, int d, int causal,
               float scale, void* stream);

/*
 * fa_bwd - attention backward pass, bf16 (the pass the QbitAI
 * FlashAttention-3 article times beside the forward in its benchmark
 * section; its arithmetic is the chain rule through the softmax).
 *
 * For O = softmax(scale * Q K^T) V (causal mask as fa_fwd) and an upstream
 * gradient dO, writes the gradients of sum(dO * O):
 *     D_i = sum_c dO_ic O_ic,   P = exp(scale * Q K^T - LSE) (masked: 0)
 *     dV = P^T dO,   dS = P * (dO V^T - D),
 *     dQ = scale * dS K,   dK = scale * dS^T Q.
 * P is recomputed tile by tile from the forward's LSE; no N x N matrix is
 * stored. Each gradient row is written by exactly one workgroup (no atomics:
 * results are bitwise reproducible run to run).
 *
 * q, k, v, o, dout : bf16 [B, H, N, d] (inputs; o and lse are what fa_fwd
 *                    returned for the same q, k, v, causal and scale)
 * lse              : float32 [B, H, N] (input, required)
 * dq, dk, dv       : bf16 [B, H, N, d] (outputs; must not alias the inputs)
 * d                : 64, 96, 128 or 256
 * Arithmetic: bf16 matrix-core products with float32 accumulation; P and dS
 * are rounded to bf16 as operands of the second products; D is a float32 sum.
 * Scratch: 2 * B*H*N floats, stream-ordered from the library's pool.
 * Validation order: null q/k/v/o/lse/dout/dq/dk/dv -> INVALID_ARG; B, H or
 * N < 1 -> INVALID_ARG; d not in {64, 96, 128, 256} -> UNSUPPORTED; scale not
 * finite and > 0 -> INVALID_ARG; N*d > 2^30, B*H >= 2^31 or
 * B*H*ceil(N/128) >= 2^24 (the grid limit of 2^32 - 1 work-items) ->
 * TOO_LARGE; a pointer not 16-byte aligned -> MISALIGNED; launch or scratch
 * allocation error -> HIP.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const float* lse, const void* dout, void* dq, void* dk, void* dv,
           int B, int H, int N, int d, int causal, float scale, void* stream);

/*
 * fa_fwd_splitkv - attention forward with the key axis split across
 * workgroups (FlashDecoding: parallelise over the key/value length for
 * decode; droidorbit FlashAttention-3 explainer, FAQ on FlashDecoding).
 *
 * q : bf16 [B, H, Nq, d]       k, v : bf16 [B, H, Nk, d]
 * o : bf16 [B, H, Nq, d]       lse  : float32 [B, H, Nq] or NULL
 * d : 64, 96 or 128.   scale : finite > 0.
 * causal != 0: the queries are the last Nq of the Nk positions, so query i
 *   attends keys j <= i + Nk - Nq (needs Nq <= Nk). With Nq == Nk this is
 *   fa_fwd's mask.
 * num_splits : 0 = automatic: for Nq <= 32 (decode) enough splits for two
 *   workgroups per compute unit twice over, at least two 64-key tiles each;
 *   for longer queries a split only when B*H*ceil(Nq/128) < 256: about 512
 *   (query tile, split) items with at least eight tiles each, or, causal,
 *   about 768 items, at most 8 splits, at least four tiles each. Else the
 *   number of splits (capped at ceil(Nk/64)). The count used is
 *   fa_splitkv_splits().
 * Each split's workgroups write a float32 partial output and log-sum-exp to
 * stream-ordered scratch from the library's pool (splits * B*H*Nq * (d+1)
 * floats); a second kernel merges them:
 *   LSE = log sum_s exp(LSE_s),  O = sum_s exp(LSE_s - LSE) O_s  -> bf16.
 * The products are the forward's (bf16 operands, fp32 accumulation, P in
 * bf16); the result differs from fa_fwd's only by rounding order.
 * Validation order: null q/k/v/o -> INVALID_ARG; B, H, Nq or Nk < 1, or
 * num_splits < 0 -> INVALID_ARG; causal with Nq > Nk -> INVALID_ARG; d not in
 * {64, 96, 128} -> UNSUPPORTED; scale not finite and > 0 -> INVALID_ARG;
 * Nk*d > 2^30, Nq*d > 2^29, B*H >= 2^31, or either launch above 2^32 - 1
 * work-items (split kernel: 64 threads per 32 queries per split; merge: d/4
 * threads per query row) -> TOO_LARGE; a pointer not 16-byte aligned ->
 * MISALIGNED; launch or scratch allocation error -> HIP.
 */
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int Nq, int Nk, int d, int causal, float scale,
                   int num_splits, void* stream);

/*
 * fa_fwd_splitkv_noalloc - fa_fwd_splitkv for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving (decode) loops,
 * harnesses that forbid allocation. Same arguments, kernels, split count and
 * result (bit for bit) as fa_fwd_splitkv; it calls no allocator. Its scratch
 * (the partial outputs and log-sum-exps, splits * B*H*Nq * (d+1) floats) is
 * a fixed array of FA_NOALLOC_SCRATCH_BYTES bytes in device memory that each
 * device the library runs on holds until the process ends; its address is
 * looked up on the first call on a device. The caller still provides q, k,
 * v, o and lse.
 * All calls on one device share that device's array: calls that overlap on
 * one device (different streams or threads, or a captured graph replayed
 * while another call runs) race and must be serialised by the caller. Every
 * partial the merge reads is written by the same call, so nothing needs
 * clearing between calls.
 * Validation order: as fa_fwd_splitkv, then a scratch need above
 * FA_NOALLOC_SCRATCH_BYTES -> SCRATCH_LIMIT (before the alignment check).
 */
#define FA_NOALLOC_SCRATCH_BYTES (32u << 20)
int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int Nq, int Nk, int d, int causal, float scale,
                           int num_splits, void* stream);

/* The number of splits fa_fwd_splitkv uses for these sizes (causal and
 * num_splits as passed to it); INVALID_ARG for sizes < 1 or num_splits < 0.
 * Host only. */
int fa_splitkv_splits(int B, int H, int Nq, int Nk, int causal, int num_splits);

/* Human-readable text for a status code (static storage, never NULL). */
const char* fa_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
