/*
 * kamera.h — C ABI of libkamera.so, the Kamera KV reuse operator for AMD MI355X (gfx950).
 *
 * The operator (technical summary of "Kamera: Unified Position-Invariant Multimodal KV Cache
 * for Training-Free Reuse", §2 Methodology, the reuse equation):
 *
 *     KV^(B|A) = R(delta) . KV(B|empty) + U_m V_m^T
 *
 *   - KV(B|empty) is a chunk's canonical, position-free KV: keys carry RoPE at chunk-local
 *     positions 0..n_tokens-1, so one shift delta moves every token of the chunk.
 *   - R(delta) is the exact RoPE phase shift of the keys to the new position (same section:
 *     relocation is an algebraic rotation, not a forward pass). Values are not rotated.
 *   - U_m V_m^T is the rank-m conditioning patch (same section, its rank-m patch subsection),
 *     added after the rotation, in the target frame, to both channels.
 *   - GQA and MHA rotate the whole key; MLA rotates only the 64-dim k_rope and reuses c_KV
 *     unchanged (same section, "Unified Architecture Support"; the Irminsul abstract on the
 *     authors' publication page gives the same delta-rotation rule for k_r).
 *
 * Channels. Every model has two channels:
 *   channel 0 (KAMERA_CH_ROT)   GQA/MHA keys, or MLA k_rope: rotated by R(delta), then patched;
 *   channel 1 (KAMERA_CH_PLAIN) GQA/MHA values, or MLA c_KV: not rotated, then patched. With
 *                               m = 0 this channel is moved bit for bit (integer copy).
 *
 * Element types. KAMERA_DTYPE_F32 or KAMERA_DTYPE_BF16; canonical KV, patch factors and the
 * cache all use the model's type. Arithmetic is fp32; cos/sin(delta*theta_i) are formed in
 * fp64 on the device and rounded to fp32 once; the result is rounded once (RNE) on store.
 *
 * Memory. Every tensor pointer in these structs is device memory owned by the caller. The
 * structs themselves and the chunk array are host memory, read only during the call. The
 * library never allocates device memory: the caller passes a workspace of at least
 * kamera_workspace_bytes(n_chunks) bytes (device memory, 256-byte aligned), into which each
 * call copies its job table.
 *
 * Staging. That copy starts from a per-device ring of pinned host memory (32 MiB, 256 calls in
 * flight), the library's only allocation: made once per device by kamera_init(), or by the
 * first compute call on a device that was not initialised. A compute call never allocates or
 * frees after that and never blocks the host: when every ring region it could use still feeds
 * a copy the device has not reached, it returns KAMERA_ERR_BUSY having enqueued nothing
 * (synchronise the stream, or let it progress, and call again). A table larger than the ring
 * (a batch of more than ~70,000 chunks) is KAMERA_ERR_UNSUPPORTED.
 *
 * Streams. The compute calls enqueue work on `stream` (a hipStream_t; NULL = default stream)
 * and return without synchronising. A device fault surfaces at the caller's next sync. The
 * workspace must not be reused by another call until this call's work has finished on the
 * stream (calls on one stream serialise by themselves). A stream that is being captured into
 * a graph is rejected (KAMERA_ERR_UNSUPPORTED): the captured copy would replay from a ring
 * region that later calls reuse.
 *
 * Errors. Compute calls validate every argument on the host before anything is enqueued; on
 * any error they return a status != KAMERA_OK, enqueue nothing, and set a per-thread message
 * readable with kamera_last_error(). No C++ exception crosses this ABI.
 *
 * Thread safety. Calls are reentrant. Mutable global state: the per-thread error message and
 * the per-device staging rings (each guarded by its own mutex, held only while a call claims a
 * region; kept until the process ends).
 */
#ifndef KAMERA_H_
#define KAMERA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KAMERA_VERSION 10300 /* major*10000 + minor*100 + patch */

typedef enum kamera_status {
  KAMERA_OK = 0,
  KAMERA_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative size, inconsistent geometry */
  KAMERA_ERR_UNSUPPORTED = 2,      /* valid but not implemented (dtype, head width, m > 256) */
  KAMERA_ERR_OVERLAP = 3,          /* a chunk's source range overlaps the destination pool */
  KAMERA_ERR_WORKSPACE = 4,        /* workspace missing, misaligned or too small */
  KAMERA_ERR_HIP = 5,              /* a HIP runtime call failed (message holds its text) */
  KAMERA_ERR_BUSY = 6              /* every staging region is still in flight; nothing enqueued */
} kamera_status;

typedef enum kamera_family {
  KAMERA_FAMILY_GQA = 0, /* GQA and MHA (MHA is GQA with n_kv_heads == n_q_heads) */
  KAMERA_FAMILY_MLA = 1  /* latent c_KV (head_dim wide) + decoupled k_rope (rope_dim wide) */
} kamera_family;

typedef enum kamera_dtype { KAMERA_DTYPE_F32 = 0, KAMERA_DTYPE_BF16 = 1 } kamera_dtype;

/* Which features form a RoPE pair. HALF_SPLIT: (i, i + rot/2). INTERLEAVED: (2i, 2i + 1).
 * Pair i turns by angle delta * theta^(-2i/rot); a pair (x, y) becomes
 * (x cos - y sin, y cos + x sin); positive delta moves the chunk later. */
typedef enum kamera_rope_layout {
  KAMERA_ROPE_HALF_SPLIT = 0,
  KAMERA_ROPE_INTERLEAVED = 1
} kamera_rope_layout;

enum { KAMERA_CH_ROT = 0, KAMERA_CH_PLAIN = 1, KAMERA_N_CHANNELS = 2 };

#define KAMERA_MAX_RANK 256

#define KAMERA_MAX_SECTIONS 3

/* Model geometry.
 *   GQA/MHA: n_kv_heads heads per channel, each head_dim wide. The first rope_dim features of
 *            every key head carry RoPE (even, <= head_dim); the others pass through unchanged
 *            (partial rotary, as GPT-NeoX-style models apply it; rope_dim == head_dim rotates
 *            the whole key). bf16 heads take the MFMA path when rope_dim is 64 or 128 and
 *            head_dim - rope_dim is a multiple of 64; other even shapes up to 512 take the
 *            VALU path.
 *   MLA:     n_kv_heads must be 1; channel 1 (c_KV) is head_dim wide (kv_lora_rank, e.g. 512),
 *            channel 0 (k_rope) is rope_dim wide (e.g. 64).
 * Frequencies: pair i turns by its shift times inv_freq[i]; inv_freq == NULL means the plain
 * ladder theta^(-2i/rope_dim). A table carries model-specific frequencies (llama3, yarn,
 * linear scaling ...). The table is host memory, rope_dim/2 finite values >= 0, read during
 * the call only.
 * Multimodal positions (M-RoPE): n_sections > 0 gives each pair the position component it
 * encodes, pair_section[i] in [0, n_sections) (host memory, rope_dim/2 entries; contiguous
 * sections as in Qwen2-VL, interleaved as in Qwen3-VL). Pair i then turns by the chunk's shift
 * of that component (kamera_chunk.delta for section 0, delta_sections[s-1] for s >= 1). A
 * chunk moved along the sequence shifts every component alike, which is plain RoPE
 * relocation; sections matter when the components move by different amounts. */
typedef struct kamera_model {
  int32_t family;      /* kamera_family */
  int32_t dtype;       /* kamera_dtype */
  int32_t n_layers;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t rope_dim;
  int32_t rope_layout; /* kamera_rope_layout */
  int32_t n_sections;  /* 0: one position per token; 1..KAMERA_MAX_SECTIONS: see above */
  double rope_theta;   /* RoPE base, > 1 and finite (unused when inv_freq is given) */
  const double* inv_freq;       /* host: rope_dim/2 frequencies, or NULL */
  const uint8_t* pair_section;  /* host: rope_dim/2 section indices; NULL iff n_sections == 0 */
} kamera_model;

/* Paged destination cache, one pool per channel (for MLA both pools may live in one
 * allocation: pool[1] = rows base (c_KV), pool[0] = rows base + head_dim (k_rope)).
 * Element (layer l, physical page P, slot s, head h, feature f) of channel c is at
 *     pool[c] + l*layer_stride + (P*page_size + s)*token_stride + h*width_c + f
 * (in elements), width_c = head_dim, or rope_dim for MLA channel 0.
 * Logical token p of the cache lives in physical page page_table[p / page_size], slot
 * p % page_size. page_table == NULL means the identity table (a dense cache).
 * Table entries outside [0, n_pages) are never written through: the rows they address are
 * skipped and counted (kamera_read_fault_count).
 * Debug mode: with the environment variable KAMERA_VALIDATE set to a non-zero integer, the
 * reuse-operator calls (kamera_reuse_batch, kamera_reuse_batch_noalloc, kamera_relocate,
 * kamera_patch) first copy the page table to the host, after the stream's earlier work, and
 * synchronise the stream: a batch that writes through an entry outside [0, n_pages), or whose
 * tokens land twice on one physical slot (two logical pages sharing a physical page), is then
 * rejected with KAMERA_ERR_INVALID_ARGUMENT before anything is enqueued. In this mode the
 * calls block the host and return KAMERA_ERR_UNSUPPORTED on a capturing stream. */
typedef struct kamera_cache {
  void* pool[2];
  int64_t layer_stride;       /* elements */
  int64_t token_stride;       /* elements between consecutive slots */
  const int32_t* page_table;  /* device memory, n_logical_pages entries, or NULL */
  int32_t n_logical_pages;    /* logical pages addressable through the table */
  int32_t page_size;          /* tokens per page, > 0 */
  int32_t n_pages;            /* physical pages per layer in each pool */
  int32_t reserved0;
} kamera_cache;

/* Canonical rows of one chunk, one channel. Element (layer l, token t, head h, feature f) is at
 *     ptr + l*layer_stride + t*token_stride + h*width_c + f   (elements). */
typedef struct kamera_src {
  const void* ptr;
  int64_t layer_stride;
  int64_t token_stride;
} kamera_src;

/* Rank-m patch of one chunk, one channel: per layer and head, U (n_tokens x m) and
 * V (width_c x m), both with rows m-contiguous:
 *     U(l, h, t, r) at U + l*u_layer_stride + h*u_head_stride + t*m + r
 *     V(l, h, f, r) at V + l*v_layer_stride + h*v_head_stride + f*m + r
 * The patch adds sum_r U(l,h,t,r) * V(l,h,f,r) to output element (l, t, h, f).
 * m = 0 means no patch (U and V are then ignored and may be NULL). */
typedef struct kamera_patch_ref {
  int32_t m;
  int32_t reserved0;
  const void* U;
  int64_t u_layer_stride;
  int64_t u_head_stride;
  const void* V;
  int64_t v_layer_stride;
  int64_t v_head_stride;
} kamera_patch_ref;

/* One chunk: its canonical source, the shift, where it lands and its patch per channel. */
typedef struct kamera_chunk {
  int32_t n_tokens;          /* >= 0; 0 is a no-op */
  int32_t dst_token_offset;  /* logical cache token of the chunk's token 0, >= 0 */
  int64_t delta;             /* target position minus canonical position, |delta| < 2^31
                                (section 0's shift when the model has sections) */
  int64_t delta_sections[2]; /* shifts of sections 1 and 2 (read only when n_sections > 1) */
  kamera_src src[2];         /* per channel */
  kamera_patch_ref patch[2]; /* per channel */
} kamera_chunk;

/* Sets up the current device's staging ring (see "Staging" above). Idempotent; returns
 * KAMERA_ERR_HIP if the pinned allocation fails. Call it once per device before timed or
 * latency-critical work so that no compute call makes the allocation. */
kamera_status kamera_init(void);

/* Bytes of workspace the compute calls need for n_chunks chunks (0 if n_chunks < 0). */
size_t kamera_workspace_bytes(int32_t n_chunks);

/* The reuse operator (reuse equation above) for every chunk, both channels, all layers:
 *     dst(l, p, h, :) = R(delta) src(l, t, h, :) + U V^T   with p = dst_token_offset + t.
 * Serves reuse, reorder (same patch, another delta), sliding-window survival (m = 0) and
 * recall (a fresh patch) — the three window operations of §3 — in one launch, whatever mix of
 * delta and m the chunks carry. Chunks must not write the same cache token (results would
 * race). src must not overlap the destination pools (KAMERA_ERR_OVERLAP). */
kamera_status kamera_reuse_batch(const kamera_model* model, const kamera_cache* cache,
                                 const kamera_chunk* chunks, int32_t n_chunks, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* kamera_reuse_batch for callers that cannot allocate (code that must not call hipMalloc or
 * hipFree: tight serving loops, harnesses that forbid allocation). Same validation, kernels and
 * results (bit for bit), but no workspace argument: the job tables go to a device array of
 * fixed size inside the library, one per GPU, kept until the process ends. The call allocates
 * nothing and frees nothing, and never blocks the host (KAMERA_ERR_BUSY as for the other
 * calls).
 *   Needs kamera_init() on the current device first (it locates the array and sets up the
 *   staging ring); otherwise KAMERA_ERR_UNSUPPORTED and nothing is enqueued.
 *   Limit: 1932 chunks per call (1 MiB of tables); more is KAMERA_ERR_UNSUPPORTED.
 *   Every call on one GPU reuses that GPU's array: calls whose work may overlap on the device
 *   (different streams with no ordering between them) race; calls on one stream are ordered.
 *   Rows skipped for an out-of-range page-table entry are counted in the array and are not
 *   readable (kamera_read_fault_count reads a caller's workspace). */
kamera_status kamera_reuse_batch_noalloc(const kamera_model* model, const kamera_cache* cache,
                                         const kamera_chunk* chunks, int32_t n_chunks,
                                         void* stream);

/* Relocation only, R(delta) with no patch (patch fields are ignored). Bit-identical to
 * kamera_reuse_batch with every m set to 0; channel 1 is then an exact bit copy. */
kamera_status kamera_relocate(const kamera_model* model, const kamera_cache* cache,
                              const kamera_chunk* chunks, int32_t n_chunks, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Patch only, in place on the destination: dst = round(dst + U V^T). src, delta are ignored.
 * kamera_relocate then kamera_patch may differ from the fused kamera_reuse_batch by one
 * rounding of the intermediate (one ulp of the element type). */
kamera_status kamera_patch(const kamera_model* model, const kamera_cache* cache,
                           const kamera_chunk* chunks, int32_t n_chunks, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Rows skipped since the workspace was last set up because their page-table entry was outside
 * [0, n_pages). Synchronises `stream`. Returns KAMERA_ERR_INVALID_ARGUMENT on NULL args. */
kamera_status kamera_read_fault_count(const void* workspace, void* stream, uint32_t* count);

/* Bytes of one chunk's patch factors (U and V, both channels, all layers and heads) for a
 * chunk of n_tokens tokens at rank m, in the model's element type; 0 on invalid input.
 * Patch-footprint helper (technical summary §4, "Efficiency: Memory"). */
size_t kamera_patch_bytes(const kamera_model* model, int32_t n_tokens, int32_t m);

/* Bytes of one chunk's canonical KV (both channels, all layers); 0 on invalid input. */
size_t kamera_kv_bytes(const kamera_model* model, int32_t n_tokens);

/* ---- Patch compile ------------------------------------------------------------------------
 * The technical summary (§2) forms each chunk's patch once, from one conditioned pass over
 * [A, B]: the deficit Delta = KV(B|A) - R(delta) KV(B|empty) (the deficit of §1, taken in the
 * frame of the conditioned pass) is reduced to its top-m factors by SVD. kamera_patch_compile
 * takes KV(B|A) as given (the forward pass that produces it is outside this library) and writes
 * per layer and head
 *     V (width x m): an orthonormal basis of Delta's top-m right singular subspace,
 *     U (n_tokens x m) = Delta V,
 * so that U V^T is the best rank-m approximation of Delta (Eckart-Young) once the subspace
 * iteration has converged. Factors are written in the model's element type and can be passed
 * to kamera_reuse_batch as they are. Method on the device: G = Delta^T Delta (fp32 MFMA), block
 * power iteration on G from a fixed start with CholeskyQR2 re-orthonormalisation (n_iter
 * rounds), then U = Delta V. Singular values are not returned; U carries them. */

/* Where kamera_patch_compile writes one channel's factors (device memory, model element type):
 *     U(l, h, t, r) at U + l*u_layer_stride + h*u_head_stride + t*m + r
 *     V(l, h, f, r) at V + l*v_layer_stride + h*v_head_stride + f*m + r */
typedef struct kamera_factors_out {
  void* U;
  int64_t u_layer_stride;
  int64_t u_head_stride;
  void* V;
  int64_t v_layer_stride;
  int64_t v_head_stride;
} kamera_factors_out;

/* One chunk to compile: its canonical KV(B|empty), its conditioned KV(B|A) (same layout rules
 * as kamera_src), the shift delta between the two (position of the chunk in the conditioned
 * pass minus its canonical position), the rank m (both channels) and the output factors.
 * Supported: rotated channel width a multiple of 32 up to 128; unrotated width that, or a
 * multiple of 128 up to 512; a partially rotary head with rope_dim a multiple of 16 and
 * head_dim - rope_dim a multiple of 8; m in [1, 64], m <= width, and m <= 32 for widths above
 * 128. Input rows must start on 16-byte boundaries (pointer and strides), else
 * KAMERA_ERR_UNSUPPORTED.
 * A chunk with n_tokens == 0 is skipped and its outputs are not written. Where Delta offers
 * fewer than m independent directions (Delta = 0, n_tokens < m), the surplus columns of V are
 * zero or directions on which Delta vanishes to rounding, and U's columns there are ~0. */
typedef struct kamera_compile_chunk {
  int32_t n_tokens;
  int32_t m;
  int64_t delta;              /* as in kamera_chunk */
  int64_t delta_sections[2];  /* as in kamera_chunk */
  kamera_src canonical[2];
  kamera_src conditioned[2];
  kamera_factors_out out[2];
} kamera_compile_chunk;

#define KAMERA_COMPILE_MAX_RANK 64

/* Bytes of workspace kamera_patch_compile needs for these chunks (fp32 Gram matrices and bases
 * of every layer and head, plus the job table); depends only on the model and each chunk's
 * n_tokens and m (pointers are not read). 0 if the arguments are invalid or unsupported
 * (kamera_last_error() says which check failed). */
size_t kamera_compile_workspace_bytes(const kamera_model* model,
                                      const kamera_compile_chunk* chunks, int32_t n_chunks);

/* Compile the patches of `chunks` (see above) on `stream`. n_iter: rounds of subspace
 * iteration, 1..100 (8 is plenty when the deficit's spectrum drops by 10x after rank m).
 * The extent of every U and V must be disjoint from every other output's and from every input's
 * extent (KAMERA_ERR_OVERLAP). Results are deterministic and do not depend on which other
 * chunks share the call. Same validation, stream and error conventions as the compute calls. */
kamera_status kamera_patch_compile(const kamera_model* model, const kamera_compile_chunk* chunks,
                                   int32_t n_chunks, int32_t n_iter, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* ---- Orbit patch ------------------------------------------------------------------------
 * One patch for every ordering of a cached set (technical summary §3, the reorder window
 * operation: a single patch, averaged over permutations, serves every ordering). The caller
 * lists, per chunk, the orderings to average: for each, the chunk's conditioned KV in that
 * ordering (KV(B | its predecessors there), from the caller's forward pass) and its shift.
 * The deficits are averaged, each in its own frame,
 *     Delta_bar = (1/K) sum_k [ KV_k(B|A_k) - R(delta_k) KV(B|empty) ],
 * and Delta_bar is reduced exactly as kamera_patch_compile reduces Delta (same factors, same
 * limits, same outputs). On the device the mean of the rotations acts on each pair as
 * [[mean cos, -mean sin], [mean sin, mean cos]] (fp64 means, one rounding), so each streaming
 * pass reads the canonical rows once and every ordering's conditioned rows once. With one
 * ordering the result is bit-identical to kamera_patch_compile. */
#define KAMERA_ORBIT_MAX_MEMBERS 64

typedef struct kamera_orbit_member {
  int64_t delta;              /* the chunk's position in this ordering minus its canonical one */
  int64_t delta_sections[2];  /* as in kamera_chunk */
  kamera_src conditioned[2];  /* per channel; same layout rules as kamera_src */
} kamera_orbit_member;

typedef struct kamera_orbit_chunk {
  int32_t n_tokens;
  int32_t m;
  int32_t n_members;                   /* orderings averaged, 1..KAMERA_ORBIT_MAX_MEMBERS */
  int32_t reserved0;
  const kamera_orbit_member* members;  /* host, n_members entries, read during the call */
  kamera_src canonical[2];
  kamera_factors_out out[2];
} kamera_orbit_chunk;

/* Workspace bytes for kamera_patch_compile_orbit (geometry only); 0 on invalid arguments. */
size_t kamera_orbit_compile_workspace_bytes(const kamera_model* model,
                                            const kamera_orbit_chunk* chunks, int32_t n_chunks);

/* The orbit patch of every chunk (see above), on `stream`. Validation, overlap rules (every
 * member's conditioned rows are inputs), n_iter and error conventions as kamera_patch_compile. */
kamera_status kamera_patch_compile_orbit(const kamera_model* model,
                                         const kamera_orbit_chunk* chunks, int32_t n_chunks,
                                         int32_t n_iter, void* workspace, size_t workspace_bytes,
                                         void* stream);

/* ---- Consumer side: decode attention and the state merge ----------------------------------
 * The abstract states that the direct readout of a cached chunk is recovered exactly by the
 * standard state merge: attention of a query over several chunks equals the log-sum-exp
 * weighted combination of its attention over each. These calls read the relocated cache.
 *
 * kamera_decode_attention: one layer of a GQA/MHA bf16 cache (head_dim 64 or 128). Query j
 * (n_q_heads heads of head_dim bf16 values at q + j*n_q_heads*head_dim, device) attends to
 * logical cache tokens [kv_start_j, kv_start_j + kv_len_j) through the page table, with
 * scores scale * <q_h, k_t>; query head h reads KV head h / (n_q_heads / n_kv_heads) (at
 * most 16 query heads per KV head). Per query head it writes
 *     out[(j*n_q_heads + h)*head_dim + f] = sum_t softmax(scores)_t v_tf      (fp32)
 *     lse[j*n_q_heads + h] = log sum_t exp(score_t)                          (fp32, natural)
 * (out = 0 and lse = -inf when kv_len == 0). The key ranges are cut into segments of 2048,
 * 1024 or KAMERA_ATTN_SEGMENT tokens (4096 too with n_kv_heads a multiple of 4), the longest
 * that still gives the call 2048 blocks (one per segment and KV head), or 512 blocks where
 * n_kv_heads is a multiple of 4 (one per segment and quad of KV heads, reading whole rows);
 * each is attended on its own (Q K^T with bf16 MFMA, exact products; scores in base 2, the
 * fp32 dot product times scale log2(e) rounded once to fp32, weights 2^(s - max) from the
 * hardware exp2; the weights stay fp32 for P V, fp32 MFMA) and the segments are combined with
 * the state merge, so results depend on the call's total work only at fp32 rounding level.
 * scale and scale log2(e) must be finite in fp32. Tokens whose page table entry lies
 * outside [0, n_pages) are left out (masked).
 * An MLA cache (kv_lora_rank head_dim = 512, rope_dim = 64, one latent row per token shared
 * by every query head, up to 16 query heads) is read in the absorbed form: query rows are
 * [q_c (512) | q_r (64)] (576 bf16 values per head), scores scale * (<q_c, c_KV_t> +
 * <q_r, k_rope_t>) with c_KV from pool[1] and k_rope from pool[0], and out holds the 512-wide
 * latent readout sum_t softmax(scores)_t c_KV_t per head (the caller's up-projection
 * follows). */
typedef struct kamera_attn_query {
  int32_t kv_start;  /* first logical cache token attended, >= 0 */
  int32_t kv_len;    /* tokens attended, >= 0 */
} kamera_attn_query;

/* Shortest key segment one block of kamera_decode_attention attends (calls with enough work
 * take 1024, 2048 or 4096). */
#define KAMERA_ATTN_SEGMENT 512

/* Workspace bytes for kamera_decode_attention (0 on invalid arguments). */
size_t kamera_attention_workspace_bytes(const kamera_model* model, int32_t n_q_heads,
                                        const kamera_attn_query* queries, int32_t n_queries);

kamera_status kamera_decode_attention(const kamera_model* model, const kamera_cache* cache,
                                      int32_t layer, const void* q, int32_t n_q_heads,
                                      const kamera_attn_query* queries, int32_t n_queries,
                                      float scale, float* out, float* lse, void* workspace,
                                      size_t workspace_bytes, void* stream);

/* The standard state merge of n_parts attention states over disjoint key sets (device, fp32):
 *     part_out [n_parts][n_rows][head_dim], part_lse [n_parts][n_rows]
 *  -> out [n_rows][head_dim], lse [n_rows]:
 *     L = log sum_i exp(lse_i),  out = sum_i exp(lse_i - L) part_out_i.
 * Parts with lse = -inf drop out (their part_out values are not read); a row whose parts are
 * all empty gives out = 0, lse = -inf. out and lse must not overlap the inputs.
 * head_dim <= 1024; any float alignment (16-byte loads when part_out is 16-byte aligned and
 * head_dim % 4 == 0); the sums run in a fixed order (repeat calls agree bit for bit);
 * no workspace. */
kamera_status kamera_state_merge(int32_t n_parts, int32_t n_rows, int32_t head_dim,
                                 const float* part_out, const float* part_lse, float* out,
                                 float* lse, void* stream);

/* ---- Attention over chunks read in place ---------------------------------------------
 * Decode attention, one query token per sequence, over cached chunks that are never
 * relocated (the consumer side of the reuse equation, technical summary §2; chunks are
 * combined by the abstract's state merge). Each chunk keeps its canonical rows (chunk-local
 * positions 0 .. n_tokens-1, as kamera_chunk.src) and its patch, and is read as the reuse
 * operator would have written it,
 *     k'_t = R(delta) k_t + U_K(t) V_K^T,      v'_t = v_t + U_V(t) V_V^T,
 * without forming k' or v': R(delta) is orthogonal, so <q, R(delta) k> = <R(-delta) q, k>
 * (the query turns by -delta, once per chunk), the key patch adds U_K(t) . (V_K^T q) to the
 * score and the value patch adds (sum_t p_t U_V(t)) V_V^T to the output. Per query and query
 * head:  out = sum over the tokens of its chunks of softmax_t(scale <q, k'_t>) v'_t,  and lse.
 * q: [n_queries][n_q_heads][head_dim] bf16 (device); out: [n_queries][n_q_heads][head_dim]
 * fp32; lse: [n_queries][n_q_heads] fp32 (a query with no tokens gets out = 0, lse = -inf).
 * Supported: GQA/MHA bf16, head_dim 64 or 128 (RoPE as described by kamera_model: rope_dim,
 * layout, frequency table, sections), up to 16 query heads per KV head, patch ranks m in
 * [0, 64] per channel. Canonical rows, q and their strides must be 16-byte aligned.
 * Precision: the turned query and V_K^T q are fp32, split into two bf16 terms each for bf16
 * MFMA (products exact, fp32 sums); softmax and P V as in kamera_decode_attention; the value
 * patch term (sum_t p_t U_V(t)) V_V^T with exact products and fp32 sums. Chunks are cut into
 * segments as in kamera_decode_attention (segments never cross a chunk). */
typedef struct kamera_attn_chunk {
  int32_t n_tokens;
  int32_t reserved0;             /* 0 */
  int64_t delta;                 /* as kamera_chunk.delta */
  int64_t delta_sections[2];     /* as kamera_chunk.delta_sections */
  kamera_src src[2];             /* canonical K and V rows of all layers */
  kamera_patch_ref patch[2];     /* as kamera_chunk.patch; m <= 64 (0: none) */
} kamera_attn_chunk;

/* The chunks query j attends: chunks[first_chunk .. first_chunk + n_chunks). */
typedef struct kamera_chunk_query {
  int32_t first_chunk;
  int32_t n_chunks;
} kamera_chunk_query;

/* Workspace bytes for kamera_chunk_attention (0 on invalid arguments). */
size_t kamera_chunk_attention_workspace_bytes(const kamera_model* model, int32_t n_q_heads,
                                              const kamera_attn_chunk* chunks, int32_t n_chunks,
                                              const kamera_chunk_query* queries,
                                              int32_t n_queries);

kamera_status kamera_chunk_attention(const kamera_model* model, int32_t layer,
                                     const kamera_attn_chunk* chunks, int32_t n_chunks,
                                     const kamera_chunk_query* queries, int32_t n_queries,
                                     const void* q, int32_t n_q_heads, float scale, float* out,
                                     float* lse, void* workspace, size_t workspace_bytes,
                                     void* stream);

const char* kamera_status_string(kamera_status status);
const char* kamera_last_error(void); /* per-thread; "" if none */
int32_t kamera_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KAMERA_H_ */
