/*
 * qjl.h -- C ABI of libqjl: the QJL key-cache sketch and its asymmetric
 * inner-product estimator, for AMD Instinct MI355X (gfx950).
 *
 * The method: "QJL" abstract (Zandieh, Daliri, Han) on Majid Daliri's
 * scholarfeed author page.  A key k (dimension d) is projected by a random
 * m x d sketch S; only sign(S k) is kept, m bits, plus the float32 norm ||k||.
 * A query q is projected (S q) but not quantized.  The attention score
 * q.k is estimated as
 *
 *     sqrt(pi/2) * sqrt(1 + rho^2) / m * ||k|| * sum_j (2 b_j - 1) (S q)_j
 *
 * where b_j = [ (S k)_j + rho ||k|| xi_j >= 0 ] and rho is the optional
 * dither level (rho = 0: no dither).  sqrt(pi/2)/m is the constant that makes
 * the estimate unbiased for Gaussian rows; sqrt(1 + rho^2) undoes the
 * shrinkage that dither adds.
 *
 * Sketches (qjl_variant):
 *   QJL_VARIANT_DENSE  S[j][c] iid N(0, 1)  (the dense Gaussian projection of
 *                      the QJL abstract and the "Fast Quantized
 *                      Johnson-Lindenstrauss Transforms" page).
 *   QJL_VARIANT_FQJL   m/d stacked blocks  H diag(G_b) Pi_b (H/sqrt d) diag(D_b)
 *                      with Sylvester H (+-1 entries, natural order), D_b
 *                      Rademacher, Pi_b a uniform random permutation used as
 *                      a gather (Pi u)_i = u[P_b[i]], and G_b Gaussian -- the
 *                      composition of randomized Hadamard transforms with a
 *                      Gaussian second diagonal and a permutation between the
 *                      transforms ("Fast Quantized Johnson-Lindenstrauss
 *                      Transforms" page: abstract; "Key concepts", P-FQJL).
 *                      Dither (rho > 0) is the D-FQJL smoothing of the sign
 *                      quantizer on the same page, added after the transform
 *                      and before the sign.
 *   QJL_VARIANT_DFQJL  the page's first construction alone (D-FQJL): the
 *                      same blocks without the permutation, H diag(G_b)
 *                      (H/sqrt d) diag(D_b), with Gaussian dither rho > 0.
 *   QJL_VARIANT_PFQJL  the page's second construction alone (P-FQJL): the
 *                      FQJL blocks with rho = 0 (bit-identical to
 *                      QJL_VARIANT_FQJL at rho = 0 for the same seed).
 *   All three FQJL variants draw D_b and G_b from the same streams, so for
 *   one seed they differ only in the permutation and the dither.
 *
 * Every random quantity comes from SplitMix64 counter streams keyed by the
 * seed (stream 0: dense S, 1: D, 2: P, 3: G, 4: dither magnitudes, 5: dither
 * signs), so a sketch and its dither are reproducible from (seed, d, m,
 * variant, rho) alone.  The dither of coordinate j of key i is
 * rho ||k_i|| s_ij a_j: a_j = |N(j)| is drawn once with the sketch and s_ij
 * is a random sign of the key's own (one stream-5 word per 64 coordinates of
 * the key), so each key's dither is m independent standard normals.
 *
 * Layouts (all dense, row-major, no strides):
 *   K[n_keys][d], q[n_queries][d]      float32 or bfloat16 (qjl_dtype)
 *   Sq[n_queries][m]                   float32
 *   bits[n_keys][m/32]                 uint32; bit t of word w is coordinate
 *                                      32 w + t (LSB-first); bit = 1 <=> the
 *                                      (dithered) coordinate is >= 0.  Read as
 *                                      little-endian u64 words, bit t of word
 *                                      w is coordinate 64 w + t.
 *   norms[n_keys]                      float32 ||k||_2
 *   scores[n_groups][n_q][n_k]         float32
 * Group g owns key rows [g n_k, (g+1) n_k) and query rows [g n_q, (g+1) n_q)
 * (a group is one (batch, head) pair of a KV cache).
 *
 * Precision contract: bfloat16 keys and queries are projected with the
 * bfloat16 rounding of the float32 sketch (S_bf16 = RNE(S_f32)); float32
 * inputs with S_f32.  Accumulation is float32.  Keys and the queries scored
 * against them should use the same dtype so both see the same S.
 *
 * Ownership and execution:
 *   - The caller owns every device buffer (K, q, Sq, bits, norms, scores);
 *     all of them are device pointers on the sketch's device.
 *   - The library owns the sketch (host and device copies) from
 *     qjl_make_sketch to qjl_destroy_sketch.  A sketch is immutable, so
 *     concurrent calls with one sketch on different streams are safe.
 *   - The hot calls (quantize, project, score) never allocate; they enqueue
 *     kernels on `stream` (a hipStream_t; NULL = the default stream) and
 *     return.  Kernel faults surface at the caller's next synchronization.
 *   - Argument validation happens before any HIP call.  n = 0 is a no-op.
 */
#ifndef QJL_H
#define QJL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QJL_OK = 0,
  QJL_ERR_INVALID_ARGUMENT = 1, /* NULL pointer, negative count, bad enum, misaligned pointer,
                                   wrong device, m not a multiple of 32, bad rho */
  QJL_ERR_UNSUPPORTED = 2,      /* valid but outside the implemented shapes */
  QJL_ERR_OUT_OF_MEMORY = 3,    /* host or device allocation failed (qjl_make_sketch only) */
  QJL_ERR_DEVICE = 4,           /* no usable GPU, or a HIP call / kernel launch failed */
  /* Not statuses: they give the type the range of int32, so any integer a
   * caller passes to qjl_status_string is a value of the type. */
  QJL_STATUS_RANGE_MIN_ = -2147483647 - 1,
  QJL_STATUS_RANGE_MAX_ = 2147483647
} qjl_status;

typedef enum {
  QJL_VARIANT_DENSE = 0,
  QJL_VARIANT_FQJL = 1,  /* permutation, optional dither */
  QJL_VARIANT_DFQJL = 2, /* no permutation (Pi_b = I), dither rho > 0 required */
  QJL_VARIANT_PFQJL = 3  /* permutation, no dither (rho == 0 required) */
} qjl_variant;
typedef enum { QJL_DTYPE_F32 = 0, QJL_DTYPE_BF16 = 1 } qjl_dtype;

typedef struct qjl_sketch qjl_sketch; /* opaque, library-owned */

/* Limits of this library.  dense: 1 <= d <= 512;  FQJL: d a power of two in
 * [8, 256] and m a multiple of d;  both: 32 <= m <= 8192, m % 32 == 0. */
#define QJL_MAX_D 512
#define QJL_MAX_M 8192

/*
 * Draw a sketch (the random JL matrix of the QJL abstract, or the FQJL
 * composition) from `seed` on the host, upload it to the current HIP device
 * and return it in *out.  rho >= 0 is the dither level (0: none).
 * Errors: out == NULL, m % 32 != 0, m or d out of range, bad variant,
 * rho < 0 or not finite, rho == 0 for DFQJL or rho != 0 for PFQJL ->
 * INVALID_ARGUMENT / UNSUPPORTED (per the limits above); no GPU -> DEVICE; allocation failure -> OUT_OF_MEMORY.  On error
 * *out is set to NULL (when out is not NULL).
 */
qjl_status qjl_make_sketch(uint64_t seed, int32_t d, int32_t m, int32_t variant, float rho,
                           qjl_sketch **out);

/* Free a sketch.  NULL -> INVALID_ARGUMENT.  The caller must not destroy a
 * sketch while work that uses it is still queued. */
qjl_status qjl_destroy_sketch(qjl_sketch *sk);

/* Read back a sketch's parameters (any output pointer may be NULL). */
qjl_status qjl_sketch_info(const qjl_sketch *sk, uint64_t *seed, int32_t *d, int32_t *m,
                           int32_t *variant, float *rho, int32_t *device);

/*
 * Copy the sketch's effective m x d matrix (row-major) to host memory:
 * S_f32 gets the float32 matrix applied to float32 inputs, S_bf16 the
 * bfloat16 bit patterns applied to bfloat16 inputs (dense only; for FQJL the
 * float32 matrix is the explicit product of the blocks, evaluated in double
 * and rounded, and S_bf16 must be NULL).  Either pointer may be NULL.
 */
qjl_status qjl_sketch_export(const qjl_sketch *sk, float *S_f32, uint16_t *S_bf16);

/*
 * Host-only: generate the random parameters of a sketch without a GPU, into
 * caller-owned host buffers (any may be NULL).  Dense: S_f32[m*d],
 * S_bf16[m*d].  FQJL variants: D_signs[(m/d)*d] (+1/-1), perm[(m/d)*d]
 * (the identity for DFQJL), G[(m/d)*d].  Every variant: dither_mag[m], the
 * float32 magnitudes |N(j)| that a dithered sketch's keys put their own
 * random signs on (the Fast Quantized JL page's D-FQJL dither, Key
 * concepts).  Same validation as qjl_make_sketch, except that there is no
 * rho to check.
 */
qjl_status qjl_generate_sketch_host(uint64_t seed, int32_t d, int32_t m, int32_t variant,
                                    float *S_f32, uint16_t *S_bf16, int8_t *D_signs,
                                    int32_t *perm, float *G, float *dither_mag);

/*
 * Quantize n_keys keys: bits_out[i] = packed signs of S k_i (+ dither),
 * norms_out[i] = ||k_i||_2 (QJL abstract: a JL projection whose coordinates
 * are reduced to their signs; no per-block constants, one norm per key).
 * key_index_base is the global index of row 0; key i draws its dither signs
 * as key index (key_index_base + i), so a cache appended in pieces gets the
 * same bits as one quantized whole.  (Which kernel runs depends on the
 * dtype, the shape and whether K and bits_out are 16-byte aligned; calls
 * that take different kernels can differ in coordinates within float32
 * rounding of zero, never elsewhere.  The number of keys in a call selects
 * between kernels that give identical results.)
 * K: device, [n_keys][d] in `dtype`, aligned to its element size.
 * norms_out: device float[n_keys]; bits_out: device uint32[n_keys][m/32].
 * Keys are expected finite: the bits and norm of a row holding NaN or
 * infinity are unspecified (no error is raised).
 * Environment: QJL_DENSE_SCHEDULE = prefetch, rt4 or immediate selects another
 * register schedule of the dense bfloat16 quantizer for calls of more than
 * 16384 keys at m <= 256 (any other value, or none, the default); every
 * schedule gives identical bits and norms, only the time differs.
 * Errors: NULL pointers (n_keys > 0), n_keys < 0, key_index_base < 0, bad
 * dtype, misalignment, sketch of another device -> INVALID_ARGUMENT;
 * launch failure -> DEVICE.
 */
qjl_status qjl_quantize_keys(const qjl_sketch *sk, const void *K, int32_t dtype, int64_t n_keys,
                             int64_t key_index_base, float *norms_out, uint32_t *bits_out,
                             void *stream);

/*
 * Quantize new keys straight into a key cache laid out by group (the
 * decode-time append: the QJL abstract's cache of sign bits and norms grows
 * by one key per head and token).  K: device [n_groups * keys_per_group][d]
 * in `dtype`, the keys of group g in rows [g * keys_per_group,
 * (g + 1) * keys_per_group).  Key i of group g is quantized exactly as by
 * qjl_quantize_keys and written to cache row
 *     g * cache_rows_per_group + first_row + i
 * of norms_cache (device float[n_groups * cache_rows_per_group]) and
 * bits_cache (device uint32[n_groups * cache_rows_per_group][m/32]); no
 * other row is touched.  The dither key index of a key is key_index_base plus
 * its cache row, so a cache filled by appends holds the same bits as one
 * qjl_quantize_keys call over the whole cache with the same key_index_base.
 * Errors: NULL pointers (with keys to write), negative counts or indices,
 * first_row + keys_per_group > cache_rows_per_group, overflowing row counts,
 * bad dtype, misalignment, sketch of another device -> INVALID_ARGUMENT;
 * n_groups * keys_per_group >= 2^32 -> UNSUPPORTED; launch failure -> DEVICE.
 * n_groups == 0 or keys_per_group == 0 is a no-op.
 */
qjl_status qjl_quantize_keys_into(const qjl_sketch *sk, const void *K, int32_t dtype,
                                  int64_t n_groups, int64_t keys_per_group,
                                  int64_t cache_rows_per_group, int64_t first_row,
                                  int64_t key_index_base, float *norms_cache,
                                  uint32_t *bits_cache, void *stream);

/*
 * Project n_queries queries: Sq_out[i] = S q_i in float32, not quantized (the
 * QJL abstract projects the query with the same JL matrix and keeps it
 * unquantized; no dither).  q: device [n_queries][d] in `dtype`; Sq_out: device
 * float[n_queries][m].  Errors as for qjl_quantize_keys.  For a dense sketch
 * and bfloat16 queries with d % 16 == 0, m % 64 == 0 and 16-byte aligned q
 * and Sq_out, the products run on the matrix cores exactly as in the
 * quantizer (exact bf16 products, float32 sums), so projecting a key gives
 * the very signs qjl_quantize_keys stores for it.  The same holds for the
 * FQJL sketches with bfloat16 queries at d = 128, m in {128, 256, 512} and
 * 16-byte aligned q and Sq_out (first stage on the matrix cores as in the
 * quantizer).  Other cases sum in float32 in the order of their kernel.
 */
qjl_status qjl_project_query(const qjl_sketch *sk, const void *q, int32_t dtype,
                             int64_t n_queries, float *Sq_out, void *stream);

/*
 * Estimate scores[g][i][t] = sqrt(pi/2) sqrt(1+rho^2)/m * norms[g n_k + t]
 *   * sum_j (2 bit[g n_k + t][j] - 1) * Sq[g n_q + i][j]
 * for every group g, query i < n_q and key t < n_k (the asymmetric
 * estimator of the QJL abstract).  All pointers are device pointers
 * (Sq: float[n_groups*n_q][m], bits: uint32[n_groups*n_k][m/32],
 * norms: float[n_groups*n_k], scores_out: float[n_groups][n_q][n_k]).
 * Any count 0 -> no-op.  Errors: NULL pointers, negative counts,
 * misalignment (4 bytes), sketch of another device -> INVALID_ARGUMENT;
 * launch failure -> DEVICE.
 */
qjl_status qjl_score(const qjl_sketch *sk, const float *Sq, const uint32_t *bits,
                     const float *norms, int64_t n_groups, int64_t n_q_per_group,
                     int64_t n_k_per_group, float *scores_out, void *stream);

/*
 * Workspace that qjl_decode_attention needs for these sizes, in bytes
 * (*bytes_out; 0 when any count is 0).  The caller allocates it (device
 * memory, 16-byte aligned) and may reuse it across calls on one stream.
 * Errors: NULL sk or bytes_out, negative counts, d_v < 1 -> INVALID_ARGUMENT.
 */
qjl_status qjl_decode_attention_workspace_size(const qjl_sketch *sk, int64_t n_groups,
                                               int64_t n_q_per_group, int64_t n_k_per_group,
                                               int32_t d_v, size_t *bytes_out);

/*
 * Attention output of one decoding step on the estimated scores (the QJL
 * abstract: the sketched keys serve the attention over the KV cache; the
 * KIVI abstract: decoding reads the whole cache once per token):
 *   out[g][i][:] = sum_t softmax_t(softmax_scale * s[g][i][t]) * V[g n_k + t][:]
 * with s[g][i][t] the estimate of qjl_score (never written to memory on the
 * fast path).  Pass softmax_scale = 1/sqrt(d) for the usual attention.
 * Sq, bits, norms as for qjl_score; V: device [n_groups*n_k][d_v] in
 * v_dtype (values are not sketched); out: device float[n_groups][n_q][d_v];
 * workspace: device, 16-byte aligned, at least the size above (holds the
 * softmax partials when a group's keys are split over several workgroups, or
 * the scores on the plain path; with a group per compute unit or more each
 * group is one workgroup and writes out directly).  The fast
 * paths take bf16 values with d_v = 128, m of 128, 256, 512 or 1024, fewer
 * than 2^22 keys per group and 16-byte aligned bits and V (three or more
 * queries per group with m <= 512 form the weighted sums on the matrix
 * cores); other shapes give the same result through a plain path.  Calls
 * sharing one workspace must be ordered (one stream).
 * n_groups == 0 or n_q == 0 -> no-op.  Errors: NULL pointers, negative
 * counts, n_k == 0 with n_q > 0, d_v < 1, bad v_dtype, misalignment,
 * workspace_bytes below the required size, softmax_scale not finite, sketch
 * of another device -> INVALID_ARGUMENT; launch failure -> DEVICE.
 */
qjl_status qjl_decode_attention(const qjl_sketch *sk, const float *Sq, const uint32_t *bits,
                                const float *norms, const void *V, int32_t v_dtype, int32_t d_v,
                                int64_t n_groups, int64_t n_q_per_group, int64_t n_k_per_group,
                                float softmax_scale, void *workspace, size_t workspace_bytes,
                                float *out, void *stream);

/* Bytes of device scratch the allocation-free decode attention may use on
 * each GPU (32 MiB): calls whose workspace (qjl_decode_attention_workspace_size)
 * would exceed it are rejected. */
#define QJL_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * qjl_decode_attention without a workspace argument and without any
 * allocation, for callers that cannot allocate device memory: code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments (minus the workspace), result and errors as
 * qjl_decode_attention; the workspace is a library-owned device array of
 * QJL_NOALLOC_SCRATCH_BYTES per GPU that stays allocated until the process
 * ends.  The call allocates nothing (no hipMalloc, no library allocator)
 * and only enqueues kernels on `stream`.  Every GPU has one such array and
 * each call uses all of it that it needs: calls that overlap on one GPU
 * (other streams, other threads) race and must be ordered by the caller.
 * Errors: as qjl_decode_attention; a shape whose workspace would exceed
 * QJL_NOALLOC_SCRATCH_BYTES -> UNSUPPORTED (use qjl_decode_attention with
 * a caller workspace); the scratch not found on the device -> DEVICE.
 */
qjl_status qjl_decode_attention_noalloc(const qjl_sketch *sk, const float *Sq,
                                        const uint32_t *bits, const float *norms, const void *V,
                                        int32_t v_dtype, int32_t d_v, int64_t n_groups,
                                        int64_t n_q_per_group, int64_t n_k_per_group,
                                        float softmax_scale, float *out, void *stream);

/* A static, human-readable name for a status code (never NULL). */
const char *qjl_status_string(qjl_status s);

/* Library version string, e.g. "qjl 0.1.0 gfx950". */
const char *qjl_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QJL_H */
