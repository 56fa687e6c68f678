/*
 * flashgau.h — C ABI of the FLASH layer forward pass for AMD Instinct MI355X (gfx950).
 *
 * The operation is one layer of FLASH as defined on the page "FLASH: Possibly the Most Interesting
 * Efficient Transformer Design Recently" (kexue.fm/archives/8934): a gated attention unit whose
 * token mixing is mixed-chunk attention.
 *
 *   U = SiLU(X W_u), V = SiLU(X W_v), Z = SiLU(X W_z)               ("Initial Power", eq. relu-att)
 *   Q_quad, K_quad, Q_lin, K_lin = gamma[h] ⊙ Z + beta[h], h = 0..3   ("Mixed Chunk", four heads)
 *   per chunk g of c tokens:
 *     V̂_quad_g = relu(Q_quad_g K_quad_gᵀ / c)² V_g   (entries with key j > query i zeroed if causal)
 *     V̂_lin_g  = Q_lin_g S_g / n, S_g = Σ_h K_lin_hᵀ V_h over all chunks h (non-causal) or over
 *                the earlier chunks h < g only (causal; the first chunk reads S = 0)
 *   O = [U ⊙ (V̂_quad + V̂_lin)] W_o                                  ("Mixed Chunk", last display)
 *
 * Normalisation readings (the page's constants conflict): the local term uses relu²(q·k / c), the
 * appendix convention of "Weak Attention" applied per chunk; the global term divides by the
 * sequence length n in both the causal and the non-causal form ("Extended Thoughts" says the
 * appendix divides by n). SiLU is used for Z as for U and V.
 *
 * Conventions shared by every entry point
 *   - All tensors are dense row-major; every device pointer is memory owned by the caller.
 *   - The library never allocates, frees or synchronises. Its only mutable global state is the
 *     per-device address of flash_gau_forward_noalloc's scratch array, set once per device, and
 *     a small host-side cache of the backward's split plans per shape (mutex-guarded; it changes
 *     no result, only how soon a plan is found).
 *   - flash_gau_forward enqueues its kernels on `hip_stream` (NULL = the null stream) and returns
 *     at once. Faults inside a kernel surface at the caller's next synchronisation.
 *   - Every argument is validated on the host before the first launch; on any error nothing has
 *     been launched and nothing has been written.
 *   - Sizes: B >= 0 and n >= 0 (B*n == 0 is an empty call that succeeds and launches nothing);
 *     d, e, s, chunk >= 1; n % chunk == 0; d, e, s and chunk must be multiples of 8 so that
 *     every row starts on a 16-byte boundary; every dimension and product used as a row count
 *     must fit in int32 (B*n, 2e+s, B*(n/chunk)*max(e, s)).
 */
#ifndef FLASHGAU_H
#define FLASHGAU_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage and arithmetic type of X, the weights, O and every intermediate. bf16 runs accumulate
 * in fp32 (matrix-core accumulators) and store intermediates as bf16 (round to nearest even);
 * f32 runs are fp32 throughout. gamma and beta are always fp32. */
typedef enum { FLASHGAU_F32 = 0, FLASHGAU_BF16 = 1 } flashgau_dtype;

/* Return codes. */
#define FLASHGAU_OK 0
#define FLASHGAU_ERR_NULL_PTR (-1)    /* a required pointer is NULL */
#define FLASHGAU_ERR_BAD_SHAPE (-2)   /* negative/zero size, n % chunk != 0, a size overflows, or a
                                       position / rotary base out of range */
#define FLASHGAU_ERR_UNSUPPORTED (-3) /* unknown dtype; d, e, s, chunk not a multiple of 8; or the
                                       score buffer B*n*chunk above 2^33 elements (see P below) */
#define FLASHGAU_ERR_MISALIGNED (-4)  /* a tensor pointer is not 16-byte aligned */
#define FLASHGAU_ERR_WORKSPACE (-5)   /* workspace_bytes smaller than flashgau_workspace_size() */
#define FLASHGAU_ERR_ALIASING (-6)    /* O or the workspace overlaps an input or each other */
#define FLASHGAU_ERR_HIP (-7)         /* a kernel launch was rejected by the HIP runtime */
#define FLASHGAU_ERR_TOO_LARGE (-8)   /* flash_gau_forward_noalloc: the problem's workspace exceeds
                                       its fixed scratch (flashgau_noalloc_scratch_bytes()) */

/* Workspace buffers, in the order of their byte offsets (see flashgau_workspace_offsets). Each
 * holds an intermediate of the one forward path; tests read them to check each stage. Layouts,
 * with G = n / chunk and element type = the call's dtype:
 *   WCAT_T  [2e+s, d]     transposed, concatenated projection weights (W_u | W_v | W_z)ᵀ
 *   WO_T    [d, e]        transposed output weights W_oᵀ
 *   VT      [B*G, e, c]   SiLU(X W_v), transposed inside each chunk (token index fastest)
 *   QQ, KQ, QL [B*n, s]   the heads Q_quad, K_quad, Q_lin
 *   KLT     [B*G, s, c]   the head K_lin, transposed inside each chunk
 *   P       [B*G, c, c]   relu(Q_quad K_quadᵀ / c)² per chunk. Causal: the entries above the
 *                         diagonal that the mix stage reads are zero; blocks of entries lying
 *                         entirely above the diagonal are left unwritten (never read). Every
 *                         chunk's scores are materialised, so B*n*chunk may not exceed 2^33
 *                         (16 GiB in bf16): a longer single chunk (FLASH-Quad, chunk = n, beyond
 *                         n = 92681 for B = 1) returns FLASHGAU_ERR_UNSUPPORTED
 *   ST      [B*G, e, s] (causal) or [B, e, s] (non-causal): the state S_g / n, transposed.
 *                         Left unwritten when causal and n == chunk (the one chunk's prefix is
 *                         empty, so the global term vanishes and its stages launch nothing)
 *   Y       [B*n, e]      U ⊙ (V̂_quad + V̂_lin), U = SiLU(X W_u) (U itself is never stored: the
 *                         mix stage computes it for its own tile)
 *   CARRY   [B, NG, e, s] per sequence, the sum of K_linᵀ V over each group of consecutive
 *                         chunks, / n, transposed. The states stage splits the n/c chunks of a
 *                         sequence into NG groups of ceil((n/c) / NG) chunks (NG is chosen from the
 *                         shape so that about two thousand workgroups run); the carry stage adds the
 *                         totals of earlier groups to every chunk's state.                        */
enum {
  FLASHGAU_WS_WCAT_T = 0,
  FLASHGAU_WS_WO_T,
  FLASHGAU_WS_VT,
  FLASHGAU_WS_QQ,
  FLASHGAU_WS_KQ,
  FLASHGAU_WS_QL,
  FLASHGAU_WS_KLT,
  FLASHGAU_WS_P,
  FLASHGAU_WS_ST,
  FLASHGAU_WS_Y,
  FLASHGAU_WS_CARRY,
  FLASHGAU_WS_COUNT
};

/* Bytes of device workspace flash_gau_forward needs for this problem. Host-only; makes no HIP
 * call. Writes the size to *out_bytes (0 for an empty problem) and returns FLASHGAU_OK, or returns
 * an error code (same validation as flash_gau_forward) and leaves *out_bytes untouched. */
int flashgau_workspace_size(int64_t B, int64_t n, int64_t d, int64_t e, int64_t s, int64_t chunk,
                            int causal, flashgau_dtype dtype, size_t* out_bytes);

/* The same size as a plain return value: bytes of device workspace flash_gau_forward needs, or 0
 * when the problem is empty (B*n == 0) or invalid (any case in which flashgau_workspace_size
 * returns an error code; call that function to tell the two apart). Host-only. */
size_t flashgau_workspace_bytes(int64_t B, int64_t n, int64_t d, int64_t e, int64_t s,
                                int64_t chunk, int causal, flashgau_dtype dtype);

/* Byte offsets of the FLASHGAU_WS_* buffers inside the workspace (each 256-byte aligned), written
 * to out_offsets[0 .. FLASHGAU_WS_COUNT-1]. Host-only. Returns FLASHGAU_OK or an error code. */
int flashgau_workspace_offsets(int64_t B, int64_t n, int64_t d, int64_t e, int64_t s,
                               int64_t chunk, int causal, flashgau_dtype dtype,
                               size_t* out_offsets);

/* Number NG of chunk groups the states stage uses for this problem (the CARRY buffer holds
 * B * NG * e * s elements). Host-only. Returns FLASHGAU_OK or an error code. */
int flashgau_state_groups(int64_t B, int64_t n, int64_t d, int64_t e, int64_t s, int64_t chunk,
                          int causal, flashgau_dtype dtype, int64_t* out_groups);

/* One FLASH layer forward, O = FLASH(X) as defined at the top of this header.
 *   X        [B, n, d]   dtype, device
 *   W_u, W_v [d, e]      dtype, device
 *   W_z      [d, s]      dtype, device
 *   gamma    [4, s]      fp32, device; rows Q_quad, K_quad, Q_lin, K_lin
 *   beta     [4, s]      fp32, device; same row order
 *   W_o      [e, d]      dtype, device
 *   chunk    c, the chunk length; causal != 0 selects the decoder (causal) form
 *   O        [B, n, d]   dtype, device; fully overwritten
 *   workspace, workspace_bytes: device scratch of at least flashgau_workspace_size() bytes;
 *            may be NULL only when that size is 0. Its contents on return are the intermediates
 *            listed above (valid once the stream has run the call).
 *   hip_stream: a hipStream_t (NULL for the null stream).
 * Every tensor pointer must be 16-byte aligned. O and the workspace must not overlap each other
 * or any input. Returns FLASHGAU_OK or one of the error codes above. */
int flash_gau_forward(const void* X, const void* W_u, const void* W_v, const void* W_z,
                      const float* gamma, const float* beta, const void* W_o, int64_t chunk,
                      int causal, int64_t B, int64_t n, int64_t d, int64_t e, int64_t s,
                      flashgau_dtype dtype, void* O, void* workspace, size_t workspace_bytes,
                      void* hip_stream);

/* flash_gau_forward with the weights packed once per weight set by flashgau_pack_weights (the
 * transposed layout every GEMM of the forward reads, declared with the decoding entry points
 * below): the call then runs no transpose. packed, packed_bytes: that buffer (at least
 * flashgau_packed_weights_size(d, e, s, dtype) bytes, 16-byte aligned, same d, e, s and dtype);
 * it must not overlap O or the workspace. The WCAT_T and WO_T regions of the workspace are left
 * unwritten. Every other argument, the validation and the result (bitwise) are as for
 * flash_gau_forward of the weights that were packed. Returns FLASHGAU_OK or an error code. */
int flash_gau_forward_packed(const void* X, const void* packed, size_t packed_bytes,
                             const float* gamma, const float* beta, int64_t chunk, int causal,
                             int64_t B, int64_t n, int64_t d, int64_t e, int64_t s,
                             flashgau_dtype dtype, void* O, void* workspace,
                             size_t workspace_bytes, void* hip_stream);

/* flash_gau_forward for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. The same kernels, the same
 * validation and the same result (bitwise) as flash_gau_forward; the workspace is instead a
 * device array inside the library, flashgau_noalloc_scratch_bytes() bytes (64 MiB) on every GPU
 * the library is loaded on, held until the process ends. A problem whose workspace
 * (flashgau_workspace_size) is larger returns FLASHGAU_ERR_TOO_LARGE before anything is launched.
 * The call makes no allocation of any kind. It uses the copy of the array on the device that
 * hip_stream belongs to (the null stream: the current device), looked up on the first call on
 * that device (hipGetSymbolAddress, with that device made current for the lookup and the current
 * device restored after it). Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (concurrent streams, or host threads) race and must be serialised by the caller. The array
 * keeps the last call's intermediates; nothing in it needs to start at zero. Arguments as for
 * flash_gau_forward, without the workspace. Returns FLASHGAU_OK or an error code. */
int flash_gau_forward_noalloc(const void* X, const void* W_u, const void* W_v, const void* W_z,
                              const float* gamma, const float* beta, const void* W_o,
                              int64_t chunk, int causal, int64_t B, int64_t n, int64_t d, int64_t e,
                              int64_t s, flashgau_dtype dtype, void* O, void* hip_stream);

/* Bytes of the fixed scratch array flash_gau_forward_noalloc uses (host-only). */
size_t flashgau_noalloc_scratch_bytes(void);

/* flash_gau_forward with a rotary position embedding of the four heads. The FLASH page
 * ("Experimental Analysis") says the paper's models use RoPE but does not define it; the reading
 * taken is the standard rotary form: after the scale and offset, the pairs (h_{2k}, h_{2k+1}) of
 * each head vector of the token at position m (its index inside its sequence, 0-based) are
 * rotated by the angle m·θ_k, θ_k = rope_base^(-2k/s) (s is a multiple of 8, so even). The
 * angles are evaluated in double precision. rope_base must be > 0 and finite (10000 is the usual
 * value); every other argument, and the workspace contents (with rotated heads), are as for
 * flash_gau_forward. */
int flash_gau_forward_rope(const void* X, const void* W_u, const void* W_v, const void* W_z,
                           const float* gamma, const float* beta, const void* W_o, int64_t chunk,
                           int causal, float rope_base, int64_t B, int64_t n, int64_t d, int64_t e,
                           int64_t s, flashgau_dtype dtype, void* O, void* workspace,
                           size_t workspace_bytes, void* hip_stream);

/* Stages of flash_gau_forward, in launch order (one kernel each). */
#define FLASHGAU_NUM_STAGES 6
/* 0 pack          : transpose W_u|W_v|W_z and W_o into the workspace (WCAT_T, WO_T)
 * 1 proj          : X W_v|W_z with SiLU and the four heads ("Initial Power", "Weak Attention")
 * 2 scores_states : one launch of two independent roles: per chunk relu(Q_quad K_quadᵀ / c)²,
 *                   masked when causal ("Mixed Chunk", local term); and K_linᵀ V summed over the
 *                   chunks of each chunk group: the exclusive prefix inside the group for every
 *                   chunk (causal) and the group total, times 1/n (none when causal, n == chunk)
 * 3 carry         : adds the totals of earlier groups to every chunk's state (causal), or sums
 *                   the group totals into the sequence's state (non-causal); launches nothing
 *                   with one group
 * 4 mix           : per chunk P V + Q_lin S / n, gated by U = SiLU(X W_u) computed in the same
 *                   workgroup ("Mixed Chunk", both terms and the gate)
 * 5 out           : Y W_o                                                                    */

/* flash_gau_forward with per-stage timing: the same validation and the same launches, and
 * stage_events points to num_events hipEvent_t handles created by the caller, in one of two forms:
 *   num_events == FLASHGAU_NUM_STAGES + 1: hipEventRecord(stage_events[i], hip_stream) right before
 *     stage i is launched and hipEventRecord(stage_events[FLASHGAU_NUM_STAGES], hip_stream) after
 *     the last stage (each interval then also holds the launch of its kernel);
 *   num_events == 2 * FLASHGAU_NUM_STAGES: stage_events[2i] and stage_events[2i + 1] record when
 *     stage i's kernel starts and ends (hipExtLaunchKernel's start and stop events); a stage that
 *     launches nothing records both at once.
 * NULL pointer or entry -> FLASHGAU_ERR_NULL_PTR, another count -> FLASHGAU_ERR_BAD_SHAPE. For an
 * empty problem no event is recorded. Used by benchmarks to time each kernel on the stream it runs
 * on. */
int flash_gau_forward_timed(const void* X, const void* W_u, const void* W_v, const void* W_z,
                            const float* gamma, const float* beta, const void* W_o, int64_t chunk,
                            int causal, int64_t B, int64_t n, int64_t d, int64_t e, int64_t s,
                            flashgau_dtype dtype, void* O, void* workspace,
                            size_t workspace_bytes, void* hip_stream, void* const* stage_events,
                            int num_events);

/* ---------------------------------------------------------------------------------------------
 * Causal decoding, one token per sequence (the RNN form).
 *
 * Page "大模型训练之加速篇 -attention优化" (blog.csdn.net), section 1.4: causal linear attention
 * can run as a recurrence over a state, the form suited to generation. Joined to the causal
 * "Mixed Chunk" layer above, token t (0-based) of chunk g = t / c, at position i = t mod c,
 * produces
 *   o_t = [u_t ⊙ (Σ_{j<=i} relu(q_quad,t · k_quad,j / c)² v_j + q_lin,t S / n)] W_o
 * where j runs over the tokens of its own chunk so far and S = Σ_{h<g} K_lin_hᵀ V_h is the state
 * of the completed chunks; after the last token of a chunk, S += K_lin_gᵀ V_g. Stepping t from 0
 * to n-1 reproduces the rows of the causal flash_gau_forward (same readings: relu²(q·k/c), /n with
 * n the normalising length, SiLU for Z). Every sequence of the batch is at the same position t.
 * ------------------------------------------------------------------------------------------- */

/* The decoder reads the weights transposed, as the forward's first stage writes them:
 * packed = [ (W_u | W_v | W_z)ᵀ  [2e+s, d] | pad to 256 B | W_oᵀ [d, e] ] in dtype.
 * flashgau_packed_weights_size: bytes of that buffer (host-only). d, e, s >= 1 and multiples of
 * 8. Returns FLASHGAU_OK or an error code. */
int flashgau_packed_weights_size(int64_t d, int64_t e, int64_t s, flashgau_dtype dtype,
                                 size_t* out_bytes);

/* Enqueues one transpose kernel that fills `packed` (packed_bytes >= the size above) from W_u,
 * W_v [d, e], W_z [d, s], W_o [e, d] on hip_stream. 16-byte aligned device pointers; `packed`
 * must not overlap the weights. Done once per set of weights, not per decoding step. */
int flashgau_pack_weights(const void* W_u, const void* W_v, const void* W_z, const void* W_o,
                          int64_t d, int64_t e, int64_t s, flashgau_dtype dtype, void* packed,
                          size_t packed_bytes, void* hip_stream);

/* The decoding state, one caller-owned device buffer holding, at the byte offsets given by
 * flashgau_decode_state_offsets (each 256-byte aligned), with element type = dtype unless noted:
 *   S   [B, s, e]  fp32   Σ K_linᵀ V over the completed chunks (not divided by n)
 *   KQ  [B, c, s]         k_quad of the current chunk's tokens 0..i (rows past i are stale)
 *   KL  [B, c, s]         k_lin of the same tokens
 *   V   [B, c, e]         v of the same tokens
 *   U   [B, e]            u of the last token (scratch of one step)
 *   QQ, QL [B, s]         q_quad, q_lin of the last token (scratch)
 *   Y   [B, e]            u ⊙ (V̂_quad + V̂_lin) of the last token (scratch)
 * The state carries everything a step needs from the earlier tokens; the step at t = 0 clears S
 * itself, so a fresh buffer needs no initialisation. One state buffer serves one stream of steps
 * at a time. */
enum {
  FLASHGAU_DS_S = 0,
  FLASHGAU_DS_KQ,
  FLASHGAU_DS_KL,
  FLASHGAU_DS_V,
  FLASHGAU_DS_U,
  FLASHGAU_DS_QQ,
  FLASHGAU_DS_QL,
  FLASHGAU_DS_Y,
  FLASHGAU_DS_COUNT
};

/* Bytes of the decoding state for B sequences (host-only). B >= 0; d, e, s >= 1 and multiples
 * of 8; chunk >= 1 with chunk + 2 s <= 8192. Returns FLASHGAU_OK or an error code. */
int flashgau_decode_state_size(int64_t B, int64_t d, int64_t e, int64_t s, int64_t chunk,
                               flashgau_dtype dtype, size_t* out_bytes);

/* Byte offsets of the FLASHGAU_DS_* buffers inside the state, written to
 * out_offsets[0 .. FLASHGAU_DS_COUNT-1] (host-only). */
int flashgau_decode_state_offsets(int64_t B, int64_t d, int64_t e, int64_t s, int64_t chunk,
                                  flashgau_dtype dtype, size_t* out_offsets);

/* One decoding step: o = the layer's output for token t of each of the B sequences.
 *   x      [B, d]  dtype, device: the tokens at position t
 *   packed, packed_bytes: weights packed by flashgau_pack_weights (same d, e, s, dtype)
 *   gamma, beta [4, s] fp32, device (rows Q_quad, K_quad, Q_lin, K_lin)
 *   chunk  c; t the position (0 <= t < n); n the normalising length of the global term
 *   rope_base: 0 for no position encoding; > 0 rotates the four heads at position t exactly as
 *          flash_gau_forward_rope does (the same base must be used for every step of a state)
 *   o      [B, d]  dtype, device; fully overwritten
 *   state, state_bytes: the decoding state (>= flashgau_decode_state_size bytes) left by the step
 *          at t - 1 of the same sequences (any contents at t = 0); updated in place
 * Steps of one state must be issued in order of t on one stream. 16-byte aligned pointers; o
 * and the state must not overlap each other or any input. B == 0 succeeds and launches nothing.
 * Returns FLASHGAU_OK or an error code (FLASHGAU_ERR_WORKSPACE when packed_bytes or state_bytes
 * is too small). */
int flash_gau_decode_step(const void* x, const void* packed, size_t packed_bytes,
                          const float* gamma, const float* beta, int64_t chunk, int64_t t,
                          int64_t n, float rope_base, int64_t B, int64_t d, int64_t e, int64_t s,
                          flashgau_dtype dtype, void* o, void* state, size_t state_bytes,
                          void* hip_stream);

/* ------------------------------------------------------------------------------ backward
 * Gradients of one FLASH layer for training. The FLASH page motivates the chunked form by its
 * parallel training ("Mixed Chunk": the causal global term stays a prefix sum over chunks) but
 * prints no gradient; these are the chain rule of the forward above for the scalar loss
 * L = Σ O ⊙ dO, with the forward's readings (local relu²(·/c), global /n, SiLU on Z, the causal
 * state of chunk g summing chunks h < g, so its gradient sums over the chunks after h).
 * The call recomputes the forward's intermediates itself (nothing has to be kept from a forward
 * call), accumulates every product in fp32 and rounds intermediates and results to dtype. */

/* Bytes of device workspace flash_gau_backward needs (host-only; same validation as
 * flash_gau_forward; 0 for an empty problem). The size is a fixed function of the arguments: it
 * includes one fp32 copy of the weight gradients per token range of their split-K sum, and the
 * range count is chosen per shape. Returns FLASHGAU_OK or an error code. */
int flashgau_backward_workspace_size(int64_t B, int64_t n, int64_t d, int64_t e, int64_t s,
                                     int64_t chunk, int causal, flashgau_dtype dtype,
                                     size_t* out_bytes);

/* Gradients of L = Σ O ⊙ dO, O = the forward (flash_gau_forward, or flash_gau_forward_rope when
 * rope_base > 0) of the same inputs:
 *   X, W_u, W_v, W_z, gamma, beta, W_o, chunk, causal: as for flash_gau_forward
 *   dO       [B, n, d]   dtype, device: the gradient arriving at the layer's output
 *   rope_base: 0 for no position encoding, > 0 as flash_gau_forward_rope (s even)
 *   dX       [B, n, d]   dtype, device
 *   dW_u, dW_v [d, e], dW_z [d, s], dW_o [e, d]   dtype, device
 *   dgamma, dbeta [4, s] fp32, device (rows Q_quad, K_quad, Q_lin, K_lin)
 *   workspace, workspace_bytes: at least flashgau_backward_workspace_size() bytes (its first
 *            flashgau_workspace_size() bytes hold the forward's intermediates, laid out as the
 *            forward's FLASHGAU_WS_* regions)
 * Every output is fully overwritten (with B == 0 or n == 0 the weight gradients are zeros).
 * Tensor pointers 16-byte aligned, gamma/beta/dgamma/dbeta 4-byte aligned. The outputs and the
 * workspace must not overlap one another or any input. Returns FLASHGAU_OK or an error code. */
int flash_gau_backward(const void* X, const void* W_u, const void* W_v, const void* W_z,
                       const float* gamma, const float* beta, const void* W_o, const void* dO,
                       int64_t chunk, int causal, float rope_base, int64_t B, int64_t n, int64_t d,
                       int64_t e, int64_t s, flashgau_dtype dtype, void* dX, void* dW_u,
                       void* dW_v, void* dW_z, float* dgamma, float* dbeta, void* dW_o,
                       void* workspace, size_t workspace_bytes, void* hip_stream);

/* Training without the backward's recompute: flash_gau_forward_train computes O exactly as
 * flash_gau_forward_rope / flash_gau_forward do (rope_base 0: none) and also leaves in the
 * workspace (at least flashgau_backward_workspace_size() bytes) everything the backward reads of
 * the forward: the projection over W_v | W_z with its pre-activations, the gate's pre-activations
 * X W_u, the heads, the scores,
 * the prefix states and the gated mix Y = U ⊙ (V̂_quad + V̂_lin). Its mix stage writes X W_u
 * rounded to the storage type and forms the gate from those rounded values, so O may differ from
 * flash_gau_forward's in the last bf16 bit (same tolerance to the exact result).
 * flash_gau_backward_saved then returns the gradients flash_gau_backward would (bitwise the same),
 * reading that workspace instead of recomputing it: it must follow a flash_gau_forward_train of
 * the same inputs, shapes and rope_base on the same stream, with the workspace untouched between.
 * Arguments, layouts, alignment and aliasing rules as flash_gau_forward / flash_gau_backward. */
int flash_gau_forward_train(const void* X, const void* W_u, const void* W_v, const void* W_z,
                            const float* gamma, const float* beta, const void* W_o, int64_t chunk,
                            int causal, float rope_base, int64_t B, int64_t n, int64_t d, int64_t e,
                            int64_t s, flashgau_dtype dtype, void* O, void* workspace,
                            size_t workspace_bytes, void* hip_stream);

int flash_gau_backward_saved(const void* X, const void* W_u, const void* W_v, const void* W_z,
                             const float* gamma, const float* beta, const void* W_o,
                             const void* dO, int64_t chunk, int causal, float rope_base, int64_t B,
                             int64_t n, int64_t d, int64_t e, int64_t s, flashgau_dtype dtype,
                             void* dX, void* dW_u, void* dW_v, void* dW_z, float* dgamma,
                             float* dbeta, void* dW_o, void* workspace, size_t workspace_bytes,
                             void* hip_stream);

/* Static, human-readable text for a return code ("unknown error" for other values). */
const char* flashgau_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* FLASHGAU_H */
