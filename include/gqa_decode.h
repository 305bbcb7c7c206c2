/*
 * gqa_decode.h -- single-query grouped-query-attention (GQA) decode on one
 * AMD Instinct MI355X (gfx950).  Plain C ABI: pointers, sizes, no C++ or
 * framework types.
 *
 * What is computed.  For every sequence s and query head i, with
 * G = h_q / h_kv query heads per KV head and KV head j = floor(i / G):
 *
 *     x_t      = scale * <q[s,i,:], K_s[t,:]>          t in [0, L_s)
 *     out[s,i] = sum_t softmax(x)_t * V_s[t,:]
 *
 * (decode-long page, "GQA fused-attention decode kernel -- long context":
 * the local attention step and "Final normalise + store"; kernel-map page,
 * VLLM_KERNEL_MAP "paged_attention_v1" for the [num_seqs, num_heads,
 * head_dim] query layout).  Each (sequence, KV head) token range is cut into
 * partitions; one workgroup per partition computes the partial triple
 * (m, l, O) of the decode-long page's tile step for all G query heads at
 * once, and a second kernel merges the partials with the page's
 * "_merge_running" rule (kernel-map page, "paged_attention_v2": per
 * partition reduce, then a cross-partition merge, fp32 max_logits and
 * exp_sum).  A sequence of at most policy.v1_max_ctx tokens is a single
 * partition and is written directly (kernel-map page, "paged_attention_v1").
 *
 * Layouts (row-major, contiguous, 16-byte aligned base pointers):
 *   q, out          [num_seqs, h_q, d_head]                    dtype
 *   paged k, v      [num_blocks, block_size, h_kv, d_head]     dtype
 *                   (gqa_decode_xsplit: the x-split layout given there)
 *   contiguous k, v [num_seqs, s_kv, h_kv, d_head]             dtype
 *   block_table     [num_seqs, max_blocks_per_seq]             int32
 *   ctx_lens        [num_seqs]                                 int32
 * Token t of sequence s lives in physical block block_table[s, t / block_size],
 * slot t % block_size.  q, k, v and out share one dtype.
 *
 * Numerics.  Q.K^T accumulates in fp32 from exact fp16/bf16 products; the
 * softmax runs in fp32 in base 2 (log2(e) folded into the scale); softmax
 * weights enter the P.V product as a two-term (hi + lo) split in the storage
 * dtype, so the weights carry about 22 (fp16) or 16 (bf16) significant bits;
 * partials and the merge are fp32; the output is rounded to nearest-even.
 *
 * Ownership.  The caller owns every buffer, the workspace included.  The
 * library never allocates, frees or synchronises; its only device state is
 * the static scratch of gqa_decode_noalloc (it also caches, per device and
 * kernel, how many workgroups fit on the device at once).  Calls on different
 * streams with distinct workspaces and outputs may run concurrently.
 *
 * Errors.  Every argument is checked on the host before any HIP call; a
 * failed check returns its status with nothing launched.  Sizes:
 * num_seqs * T_q * h_q must be below 2^30 and the longest context
 * (max_blocks_per_seq * block_size, or s_kv) at most 2^30 tokens; larger ones
 * return GQA_ERR_BAD_SHAPE.  A failed launch
 * returns GQA_ERR_LAUNCH.  Faults during execution surface at the caller's
 * next synchronisation of the stream.  Device-resident data the host cannot
 * see is handled as follows: ctx_lens[s] is clamped to
 * [0, max_blocks_per_seq * block_size]; a sequence with L_s = 0 gets a zero
 * output row; block_table entries at or past ceil(L_s / block_size) and
 * slots at or past L_s are never read; an in-range table entry that names a
 * block outside the caller's pool is undefined behaviour.
 */
#ifndef GQA_DECODE_H
#define GQA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gqa_dtype {
  GQA_F16 = 0,   /* IEEE binary16 */
  GQA_BF16 = 1   /* bfloat16 */
} gqa_dtype_t;

typedef enum gqa_status {
  GQA_OK = 0,
  GQA_ERR_NULL_PTR = 1,     /* a required pointer is NULL */
  GQA_ERR_BAD_SHAPE = 2,    /* a size is negative, zero where it may not be, or inconsistent */
  GQA_ERR_UNSUPPORTED = 3,  /* valid but not built: d_head, G, block_size or dtype */
  GQA_ERR_MISALIGNED = 4,   /* a pointer breaks the alignment stated above */
  GQA_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than gqa_decode_workspace_size(),
                               or more than gqa_decode_noalloc's static scratch */
  GQA_ERR_BAD_POLICY = 6,   /* policy fields out of range */
  GQA_ERR_BAD_SCALE = 7,    /* scale is NaN or infinite */
  GQA_ERR_LAUNCH = 8        /* the HIP runtime refused a kernel launch */
} gqa_status_t;

/*
 * Launch policy.
 *
 * partition_size == 0 selects the balanced decomposition (the MI355X
 * default): a persistent grid of as many workgroups as the device holds at
 * once, each owning an equal, 32-token-aligned share of all (sequence, KV
 * head) token ranges laid end to end.  A range that falls inside one share is
 * computed and written in one pass; a range that spans several shares is
 * split at the share boundaries and its partials are merged.  A sequence of
 * at most v1_max_ctx tokens is never split.
 *
 * partition_size > 0 (a multiple of 32, at most 1 << 20) selects the
 * kernel-map page's fixed decomposition ("paged_attention_v1" up to
 * v1_max_ctx tokens, "paged_attention_v2" with partitions of partition_size
 * tokens above it); gqa_policy_pages() gives the policy page's
 * AttentionConfig values (partition 512, threshold 8192).  Its work items are
 * (partition, group of KV heads); a single-pass sequence stays one item,
 * computed by one workgroup whose waves split its tiles and merge in LDS.  A
 * contiguous cache launches one workgroup per item; a paged cache first lists
 * its items in the workspace, largest first, and then launches no more
 * workgroups than there can be items, taking them in that order.
 *
 * v1_max_ctx >= 0.  phases selects which kernels a call launches: 0 or 3 =
 * both, 1 = partition kernel only, 2 = merge kernel only (the merge then reads
 * the partials a phase-1 call with the same arguments left in the
 * workspace); it exists so that a caller can time the two kernels apart.
 * The balanced decomposition needs num_seqs <= 7168; a larger batch uses the
 * fixed one with 512-token partitions.
 *
 * flags: 0, GQA_POLICY_FUSED_MERGE or GQA_POLICY_VALU_DOT2 (each for the
 * balanced decomposition only, and not both; other bits are errors).
 *
 * GQA_POLICY_FUSED_MERGE: the workgroup that finishes a split range last
 * merges that range itself (it finds out through a per-range atomic counter in
 * the workspace; nothing waits on anything), and no merge kernel is launched.
 * Partials pass between workgroups through device-coherent stores and loads,
 * with no device-scope fence.  It saves the merge launch, but a range's merge
 * then runs on one CU at the end of the launch, so it can pay only for batches
 * of many short split ranges (on MI355X it ties with the merge kernel on paged
 * batches and loses where ranges are long).  Contract: the workspace
 * must be zero-filled before its first call with this flag (for instance when
 * it is allocated); every call that runs to completion leaves the counters at
 * zero again, graph replays included.  phases 2 then does nothing.
 *
 * GQA_POLICY_VALU_DOT2: the partition kernel computes Q.K^T and P.V on the
 * vector ALU, as packed two-element dot products with fp32 accumulation
 * (v_dot2_f32_f16 / v_dot2_f32_bf16), instead of on the matrix cores; loads,
 * decomposition, partials and merge are unchanged.  It exists to compare the
 * two units.  Supported for d_head = 128, the contiguous and row-layout paged
 * caches and G * T_q <= 8 with the balanced decomposition; any other problem
 * returns GQA_ERR_UNSUPPORTED.  Groups of one or two KV heads get one wave
 * per head (no split of segments between waves).
 */
#define GQA_POLICY_FUSED_MERGE 1
#define GQA_POLICY_VALU_DOT2 2

typedef struct gqa_policy {
  int32_t partition_size;
  int32_t v1_max_ctx;
  int32_t phases;
  int32_t flags;           /* 0, GQA_POLICY_FUSED_MERGE or GQA_POLICY_VALU_DOT2 */
} gqa_policy_t;

/* Fill *p with the MI355X default policy. */
void gqa_policy_default(gqa_policy_t* p);
/* Fill *p with the policy page's values: partition 512, single pass up to 8192. */
void gqa_policy_pages(gqa_policy_t* p);

/*
 * Bytes of workspace gqa_decode / gqa_decode_xsplit / gqa_decode_contiguous
 * need for these sizes (max_ctx = max_blocks_per_seq * block_size, or s_kv);
 * the size covers both cache layouts.  The workspace holds the fp32 partial
 * triples (m, l, O) of split sequences (kernel-map page, "paged_attention_v2":
 * fp32 max_logits, exp_sum and partial outputs) and:
 *   balanced decomposition: one 16-byte record per (sequence, head group),
 *     plus one counter per (sequence, head group) with GQA_POLICY_FUSED_MERGE;
 *     0 bytes in all when no sequence can be split;
 *   fixed decomposition: for a paged cache, a 256-byte header and a work
 *     list of up to one 8-byte item per (sequence, KV head, partition), even
 *     when no sequence can be split (a contiguous cache needs no list).
 * h_kv is needed because records and items are counted per KV head group.
 * Its contents need no initialisation, except under GQA_POLICY_FUSED_MERGE
 * (see gqa_policy_t).  policy NULL means gqa_policy_default().
 * Returns 0 for invalid arguments.
 */
size_t gqa_decode_workspace_size(int num_seqs, int h_q, int h_kv, int d_head, int max_ctx,
                                 const gqa_policy_t* policy);

/*
 * Paged decode.  d_head in {64, 128, 256}; 1 <= G = h_q / h_kv <= 16 and h_q a
 * multiple of h_kv; block_size a power of two in [16, 256]; T_q = 1 (gqa_decode_ex takes more).
 * scale multiplies the logits (the workloads use 1 / sqrt(d_head)).  stream
 * is a hipStream_t (NULL: the default stream).  workspace may be NULL when
 * gqa_decode_workspace_size() is 0.  num_seqs == 0 returns GQA_OK and
 * launches nothing.  k_cache and v_cache must not be NULL, even when every
 * sequence is empty (the host cannot see ctx_lens): GQA_ERR_NULL_PTR.
 */
gqa_status_t gqa_decode(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_table, const int32_t* ctx_lens, void* out,
                        int num_seqs, int max_blocks_per_seq, int h_q, int h_kv,
                        int d_head, int block_size, float scale, gqa_dtype_t dtype,
                        void* workspace, size_t workspace_bytes,
                        const gqa_policy_t* policy, void* stream);

/*
 * Paged decode over the x-split cache layout (kernel-map page,
 * VLLM_KERNEL_MAP "paged_attention_v1": key_cache
 * [num_blocks, num_kv_heads, head_dim // x, block_size, x]):
 *   k_cache   [num_blocks, h_kv, d_head / 8, block_size, 8]   dtype
 *   v_cache   [num_blocks, h_kv, d_head, block_size]          dtype
 * x = 8 elements (16 bytes of fp16/bf16): element d of token slot o of KV
 * head j in block b is k_cache[b, j, d / 8, o, d % 8] and v_cache[b, j, d, o].
 * The page gives no V layout; V keeps the tokens of one d consecutive, the
 * axis the P.V product sums over, as K keeps the d of one token consecutive.
 * Everything else (arguments, block_table, ctx_lens, workspace, policy,
 * errors) is as for gqa_decode, and both give bit-identical outputs on the
 * same logical cache.
 */
gqa_status_t gqa_decode_xsplit(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* ctx_lens, void* out,
                               int num_seqs, int max_blocks_per_seq, int h_q, int h_kv,
                               int d_head, int block_size, float scale, gqa_dtype_t dtype,
                               void* workspace, size_t workspace_bytes,
                               const gqa_policy_t* policy, void* stream);

/*
 * Allocation-free paged decode, for callers that cannot allocate device
 * memory: code being captured into a HIP graph, tight serving loops, and
 * harnesses that forbid hipMalloc.  Arguments, layouts, numerics and errors
 * are those of gqa_decode, without the workspace: the partial triples and
 * range records live in a static device array of GQA_NOALLOC_SCRATCH_BYTES
 * that the library defines, one per device (each device the library runs on
 * holds it until the process ends).  The call allocates and frees nothing;
 * the caller still passes the inputs and out.
 *
 *  - The scratch needed is sized for the grid the call actually launches.
 *    With the default policy that is (2 x workgroups x heads per workgroup x
 *    G) rows of (d_head + 2) floats plus 16 bytes per (sequence, head group),
 *    about 17 MB at d_head = 128 and 34 MB at 256 on an MI355X.  A call that
 *    needs more (for instance the fixed policy of gqa_policy_pages() on a
 *    large batch) returns GQA_ERR_WORKSPACE and launches nothing.
 *  - GQA_POLICY_FUSED_MERGE returns GQA_ERR_UNSUPPORTED (its counters would
 *    have to start at zero).  Nothing else in the scratch needs clearing:
 *    every call writes the partials and records it reads.
 *  - All calls on one device share its scratch, which keeps the last call's
 *    contents (a phases = 2 call merges what the last phases = 1 call left).
 *    Calls that overlap on one device race: serialise them, for instance by
 *    issuing them on one stream.
 *  - The first call on a device looks up the scratch's device address
 *    (hipGetSymbolAddress); a failure there returns GQA_ERR_LAUNCH.
 */
#define GQA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

gqa_status_t gqa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_table, const int32_t* ctx_lens, void* out,
                                int num_seqs, int max_blocks_per_seq, int h_q, int h_kv,
                                int d_head, int block_size, float scale, gqa_dtype_t dtype,
                                const gqa_policy_t* policy, void* stream);

/*
 * Contiguous decode: every sequence holds s_kv tokens (s_kv >= 0) in a
 * [num_seqs, s_kv, h_kv, d_head] cache, one (S_kv, h_kv * d_head) row-major
 * slab per sequence as in the decode-long page's tensor-layout docstring
 * ("GQA fused-attention decode kernel -- long context"); q and out are
 * [num_seqs, h_q, d_head] (kernel-map page, "paged_attention_v1" query
 * layout).  With s_kv == 0 the output is zero and k, v may be NULL.  Same
 * rules as gqa_decode otherwise; the workspace may be NULL when
 * gqa_decode_ex_workspace_size() for this layout is 0.
 */
gqa_status_t gqa_decode_contiguous(const void* q, const void* k, const void* v, void* out,
                                   int num_seqs, int s_kv, int h_q, int h_kv, int d_head,
                                   float scale, gqa_dtype_t dtype,
                                   void* workspace, size_t workspace_bytes,
                                   const gqa_policy_t* policy, void* stream);

/*
 * Extended call: every layout and T_q >= 1 query tokens per sequence through
 * one argument block.
 *
 * T_q > 1.  The decode-long page's kernel takes Q as (T_q, h_q * d_head) per
 * sequence, loads it as G * T_q rows against the same keys and stores O as
 * (T_q, h_q * d_head); no mask is applied.  Here accordingly each of the T_q
 * query tokens of sequence s attends to all L_s keys of the cache:
 *   q, out  [num_seqs, t_q, h_q, d_head]
 *   out[s, tau, i] = sum_t softmax_t(scale * <q[s, tau, i], K_s[t]>) V_s[t]
 * The G * T_q query rows that share a KV head go through the same matrix-core
 * products, so G * t_q <= 16.  With t_q == 1 the call equals gqa_decode /
 * gqa_decode_xsplit / gqa_decode_contiguous on the same arguments.
 *
 * layout selects the cache: GQA_KV_CONTIGUOUS (k, v [num_seqs, s_kv, h_kv,
 * d_head]; s_kv used, block fields ignored), GQA_KV_PAGED (the gqa_decode
 * pools) or GQA_KV_PAGED_XSPLIT (the gqa_decode_xsplit pools; both paged
 * layouts use block_table, ctx_lens, max_blocks_per_seq and block_size).
 * Every other field, rule and error is as for those entry points; an unknown
 * layout returns GQA_ERR_UNSUPPORTED, t_q < 1 GQA_ERR_BAD_SHAPE, and
 * G * t_q > 16 GQA_ERR_UNSUPPORTED.
 */
typedef enum gqa_kv_layout {
  GQA_KV_CONTIGUOUS = 0,
  GQA_KV_PAGED = 1,
  GQA_KV_PAGED_XSPLIT = 2
} gqa_kv_layout_t;

typedef struct gqa_decode_args {
  gqa_kv_layout_t layout;
  gqa_dtype_t dtype;
  const void* q;
  const void* k;
  const void* v;
  void* out;
  const int32_t* block_table;   /* paged layouts */
  const int32_t* ctx_lens;      /* paged layouts */
  int32_t num_seqs;
  int32_t t_q;
  int32_t h_q;
  int32_t h_kv;
  int32_t d_head;
  int32_t s_kv;                 /* contiguous layout */
  int32_t max_blocks_per_seq;   /* paged layouts */
  int32_t block_size;           /* paged layouts */
  float scale;
  void* workspace;
  size_t workspace_bytes;
  const gqa_policy_t* policy;   /* NULL: gqa_policy_default() */
  void* stream;                 /* hipStream_t; NULL: the default stream */
} gqa_decode_args_t;

gqa_status_t gqa_decode_ex(const gqa_decode_args_t* args);

/* Workspace bytes gqa_decode_ex needs for *args (pointers are not read);
 * 0 when nothing can be split or the sizes are invalid. */
size_t gqa_decode_ex_workspace_size(const gqa_decode_args_t* args);

/* Static, human-readable name of a status code. */
const char* gqa_status_string(gqa_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* GQA_DECODE_H */
