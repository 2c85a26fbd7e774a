/*
 * sv_verify.h -- C ABI of the batched speculative-decoding verification
 * library for AMD Instinct MI355X (gfx950).
 *
 * The operation is the verification step of speculative decoding as the
 * spec-verify kernel card defines it (section "Method"; operand shapes from
 * "Usage" and "Requirements and limits"), batched over B independent
 * sequences:
 *
 *   greedy  - accept draft token t_i while it equals argmax of target row
 *             p_i (lowest index on ties); at the first miss emit that argmax
 *             and stop; if all K match, emit argmax of p_K.
 *   sampled - accept t_i with probability min(1, p_i(t_i)/q_i(t_i)) on
 *             row-normalised masses (rows need not be normalised: each row's
 *             mass is summed); on the first rejection draw the next token
 *             from norm(max(0, p_i - q_i)); if all K are accepted draw the
 *             bonus token from p_K.  Randomness enters only through the
 *             caller's uniforms: u_i (i < K) drives the test of t_i and u_K
 *             the single final draw, an inverse-CDF search in ascending token
 *             order returning the smallest x whose running mass exceeds
 *             u_K * (total mass).
 *
 * Every pointer argument of the verify calls is DEVICE memory owned by the
 * caller (row statistics included); the library allocates nothing and keeps
 * no pointer after returning.  Calls are asynchronous on `stream` (a
 * hipStream_t; NULL means the default stream): outputs are valid once the
 * stream has reached the call.  Between calls the library keeps only the
 * per-device properties it caches and, per workspace address, a count of the
 * calls made on it (each call tags the words it publishes in the workspace
 * with a number derived from that count); calls that share a workspace must
 * not overlap, so calls on different streams must use different workspaces.
 * Because that number is chosen on the host when the call is made, a call
 * must not be captured into a HIP graph that is replayed: every replay would
 * carry the captured number, and a replay's readers could accept words left
 * by the one before.
 *
 * Layouts (row-major, V contiguous, f32 = IEEE binary32):
 *   target_probs [B, K+1, V] f32    draft_probs [B, K, V] f32
 *   draft_tokens [B, K] int32       uniforms    [B, K+1] f32 in [0, 1)
 *   n_accepted   [B] int32 in [0,K] next_token  [B] int32 in [0, V)
 *   stats        [B, K+1] sv_row_stats (nullable)
 *
 * Preconditions that are documented, not checked on the device: all
 * probabilities finite and >= 0, every row's mass positive, uniforms in
 * [0, 1).  If they are violated the outputs are unspecified (no memory
 * outside the documented buffers is touched).  A draft token outside
 * [0, V) is defined behaviour: it is a miss (greedy) or has p(t) = q(t) = 0
 * and is rejected (sampled).
 */
#ifndef SV_VERIFY_H
#define SV_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SV_OK = 0,
    SV_ERR_INVALID_ARG = -1,  /* NULL pointer, negative size, misaligned pointer */
    SV_ERR_WORKSPACE = -2,    /* workspace NULL, misaligned or smaller than sv_workspace_size */
    SV_ERR_HIP = -3,          /* a HIP runtime call or kernel launch failed */
    SV_ERR_UNSUPPORTED = -4,  /* sizes beyond the supported maximum (V > SV_MAX_V, K > SV_MAX_K) */
    SV_ERR_SCRATCH = -5       /* the call needs more workspace than SV_SCRATCH_BYTES (no-allocation entry point) */
} sv_status;

/* Largest vocabulary and draft length the kernels accept. */
#define SV_MAX_V 524288
#define SV_MAX_K 4096

/* Bytes of the library's static device scratch, one copy per device (the
 * workspace of sv_verify_sample_batched_noalloc). */
#define SV_SCRATCH_BYTES (16u << 20)

/* Per-row statistics, one per (b, i), i in [0, K], 48 bytes.
 *   argmax, max_p : lowest index of the maximum of p_i, and that value
 *   sum_p, sum_q  : the masses P_i = sum_x p_i(x), Q_i = sum_x q_i(x)
 *   sum_min       : sum_x min(p_i(x), q_i(x))
 *   sum_pos       : sum_x max(0, p_i(x) - q_i(x))
 *   p_t, q_t      : p_i(t_i), q_i(t_i) (0 when t_i is outside [0, V))
 * Draft fields (sum_q, sum_min, sum_pos, q_t) are 0 for i == K and in greedy
 * mode; p_t is 0 for i == K.  Masses are accumulated in fp64. */
typedef struct {
    int32_t argmax;
    float max_p;
    double sum_p, sum_q, sum_min, sum_pos;
    float p_t, q_t;
} sv_row_stats;

/* Bytes of device workspace a call with these sizes needs (sampled != 0 for
 * sv_verify_sample_batched).  Returns 0 for sizes the library rejects. */
size_t sv_workspace_size(int32_t B, int32_t K, int32_t V, int32_t sampled);

/* Zero a workspace on `stream` (a fill kernel; no memset node) and restart
 * its call count.  Memory must be initialised this way before its first use
 * as a workspace, and again whenever it has held other data since it was
 * last used as one (for example a buffer freed and allocated anew at the
 * same address).  The first call on an address the library has not seen,
 * and a call with more workspace bytes than any earlier call at that
 * address, also clear it first.  Otherwise calls need no further
 * initialisation: every 255th call on a workspace clears it again on its
 * stream before it runs.
 * Errors: SV_ERR_WORKSPACE for NULL or non-16-byte-aligned memory,
 * SV_ERR_HIP when the launch fails. */
sv_status sv_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/* Greedy verification (the card's greedy bullet).  Reads target_probs and
 * draft_tokens; writes n_accepted, next_token and, when stats != NULL, the
 * row statistics (sum_p, argmax, max_p, p_t).  B == 0 is a no-op that returns
 * SV_OK without inspecting any pointer.
 * Errors (returned before anything is launched): SV_ERR_INVALID_ARG for NULL
 * buffers, B < 0, K < 0, V < 1 or pointers not 4-byte aligned;
 * SV_ERR_UNSUPPORTED for V > SV_MAX_V or K > SV_MAX_K; SV_ERR_WORKSPACE for a
 * missing or too small workspace; SV_ERR_HIP if the launch fails. */
sv_status sv_verify_greedy_batched(const float* target_probs, const int32_t* draft_tokens,
                                   int32_t B, int32_t K, int32_t V,
                                   int32_t* n_accepted, int32_t* next_token,
                                   void* workspace, size_t workspace_bytes,
                                   sv_row_stats* stats, void* stream);

/* Sampled verification (the card's speculative-sampling bullet, with the
 * "Correctness" section's unnormalised masses).  Acceptance is decided in
 * fp64 as u_i * q_i(t_i) * P_i < p_i(t_i) * Q_i; the residual is
 * w(x) = max(0, p_n(x) * Q_n - q_n(x) * P_n) (P_n * Q_n times the normalised
 * residual); if its total is 0 (rounding only) the draw uses p_n.  Same
 * errors as the greedy call. */
sv_status sv_verify_sample_batched(const float* target_probs, const float* draft_probs,
                                   const int32_t* draft_tokens, const float* uniforms,
                                   int32_t B, int32_t K, int32_t V,
                                   int32_t* n_accepted, int32_t* next_token,
                                   void* workspace, size_t workspace_bytes,
                                   sv_row_stats* stats, void* stream);

/* Sampled verification with an early exit: the outputs of
 * sv_verify_sample_batched, bit for bit (the same decisions from the same
 * partial sums), reading only what they depend on (the card's sequential
 * rule, section "Method", stops at the first rejected draft).  A sequence's
 * walks issue a row's loads only once the row two before it is accepted, so
 * they stop after the pairs 0..n+1 for a first rejection at n, and the bonus
 * row's blocks skip their loads once that rejection is published.  So a batch reads about the pairs 0..n+1 of each sequence,
 * plus row K after full acceptance, not the whole operands.  Same arguments,
 * workspace and errors as sv_verify_sample_batched, without row statistics
 * (they need every row).  Small grids that take one block per draft row read
 * every row as before. */
sv_status sv_verify_sample_early_batched(const float* target_probs, const float* draft_probs,
                                         const int32_t* draft_tokens, const float* uniforms,
                                         int32_t B, int32_t K, int32_t V,
                                         int32_t* n_accepted, int32_t* next_token,
                                         void* workspace, size_t workspace_bytes, void* stream);

/* Sampled verification on logits, warped by one temperature (the card's
 * speculative-sampling bullet holds when target and draft are warped
 * identically; here the library warps both).  target_logits [B, K+1, V] and
 * draft_logits [B, K, V] are f32 logits, finite; the warped distribution of
 * a row l is softmax(l / temperature), and verification is then that of
 * sv_verify_sample_batched on the warped rows: accept t_i iff
 * u_i * w_q(t_i) * P_i < w_p(t_i) * Q_i, with w(x) = exp((l(x) - max l) / tau)
 * (fp32) and the masses P, Q its fp64 sums; the residual and the draws use
 * the same weights.  The two weights of an acceptance test are taken with
 * fp64 range and an fp64 temperature wherever their exponent leaves
 * [-16, 0] (in fp32 they could flush to zero at a low temperature).  Every
 * weight of a row carries one factor 2^e, |e| <= half the fp32 spacing at
 * |max l| * log2(e) / tau, which cancels; results are specified for
 * |l| * log2(e) / tau below 2^30 (|e| <= 64), e.g. |l| < 10^4 at
 * tau >= 10^-4.  Beyond it the sums may overflow or vanish and the outputs
 * are unspecified (a next_token of -1 included), with no access outside the
 * arguments.  One pass over the logits: each chunk publishes its
 * maximum and its weight sum against it, and readers rescale to the row's
 * maximum.  No row statistics.  The workspace is that of the sampled call
 * (sv_workspace_size(B, K, V, 1)).  One launch on `stream`.
 * Errors: those of the sampled call, and SV_ERR_INVALID_ARG for a temperature
 * that is not finite and > 0. */
sv_status sv_verify_sample_logits_batched(const float* target_logits, const float* draft_logits,
                                          const int32_t* draft_tokens, const float* uniforms, float temperature,
                                          int32_t B, int32_t K, int32_t V,
                                          int32_t* n_accepted, int32_t* next_token,
                                          void* workspace, size_t workspace_bytes, void* stream);

/* Sampled verification on logits with an early exit: the outputs of
 * sv_verify_sample_logits_batched, bit for bit, reading only what they
 * depend on, as sv_verify_sample_early_batched does for probabilities.
 * Same arguments, workspace and errors as sv_verify_sample_logits_batched. */
sv_status sv_verify_sample_logits_early_batched(const float* target_logits, const float* draft_logits,
                                                const int32_t* draft_tokens, const float* uniforms,
                                                float temperature, int32_t B, int32_t K, int32_t V,
                                                int32_t* n_accepted, int32_t* next_token,
                                                void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the call of
 * sv_verify_sample_batched, same arguments and outputs, without a workspace.
 * Its workspace is a static device array of SV_SCRATCH_BYTES that the
 * library's code object holds on every device it runs on until the process
 * ends; the library looks up that array's address on a device at the first
 * call there (hipGetSymbolAddress) and calls no hipMalloc, hipFree or other
 * allocating routine.  Every call on one device shares that device's array
 * and finds the words the previous call left there; they carry that call's
 * tag and are ignored (the first call on a device, and every 255th after it,
 * clears the part it uses with a fill kernel on its stream).  Calls that
 * overlap on one device race on the array: issue them in order on one
 * stream, or wait between streams.  Like every call with a workspace, it
 * must not be captured into a HIP graph that is replayed.
 * Errors: those of sv_verify_sample_batched (SV_ERR_WORKSPACE excepted), and
 * SV_ERR_SCRATCH when sv_workspace_size(B, K, V, 1) > SV_SCRATCH_BYTES
 * (11.5 MB at B = 1024, K = 8, V = 128256 fits), returned before anything is
 * launched. */
sv_status sv_verify_sample_batched_noalloc(const float* target_probs, const float* draft_probs,
                                           const int32_t* draft_tokens, const float* uniforms,
                                           int32_t B, int32_t K, int32_t V,
                                           int32_t* n_accepted, int32_t* next_token,
                                           sv_row_stats* stats, void* stream);

/* Synchronously read the workspace's device-fault word into *error_out
 * (host memory), waiting for `stream` first: 0 when every call since the
 * last sv_workspace_init completed normally.  The current kernels never set
 * it: a workgroup that waits longer than its bound for another workgroup's
 * partial result computes that result itself (bit-identically), so waits
 * cannot fail. */
sv_status sv_workspace_error(const void* workspace, int32_t* error_out, void* stream);

/* Static, human-readable name of a status code. */
const char* sv_status_string(sv_status s);

#ifdef __cplusplus
}
#endif

#endif /* SV_VERIFY_H */
