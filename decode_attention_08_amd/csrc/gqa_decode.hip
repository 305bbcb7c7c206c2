// Single-query GQA decode attention for MI355X (gfx950, CDNA4).
//
// Kernels:
//   partition kernels  a workgroup holds the waves of a head group of HPW KV
//                      heads (up to 4; a group of one or two heads gets
//                      several waves per head); all its waves walk the same
//                      token segment of one sequence, so that together they
//                      read whole runs of a K/V row (the cache
//                      interleaves the KV heads of a token).  For its KV head
//                      a wave computes the partial triple (m, l, O) of the
//                      G * T_q query rows sharing it (decode-long page, "Local
//                      attention" tile sweep and "_merge_running") and either
//                      stores the normalised output (the segment is the whole
//                      sequence; kernel-map page, "paged_attention_v1") or
//                      the fp32 partial (kernel-map page, "paged_attention_v2").
//                      Two schedulers feed them: a balanced persistent grid
//                      and the pages' fixed partitions (one workgroup per
//                      item; on a paged cache a planner kernel first lists
//                      the items largest first).
//   merge kernels      1 to 64 slots of 16 lanes per (sequence, query head)
//                      of a split sequence: the n-ary form of
//                      "_merge_running" over the partials, then the
//                      decode-long page's "Final normalise + store".
//
// Matrix-core mapping (v_mfma_f32_16x16x32_{f16,bf16}, wave64).  The G * T_q
// <= 16 query rows of one KV head are the 16-wide N side of both products,
// padded with zero query rows:
//   S^T[16 tok x 16 head] += K[16 tok x 32 d] . Q^T[32 d x 16 head]
//   O^T[16 d x 16 head]   += V^T[16 d x 32 tok] . P^T[32 tok x 16 head]
// With this orientation every lane owns one head column (lane % 16) in both
// the score and the output accumulators, so the online-softmax state of a
// head never leaves its lane group; only the tile max is exchanged between
// the four 16-lane groups.  K feeds the A operand straight from HBM with
// 16-byte loads (8 consecutive d of one token per lane).  V needs tokens
// along the operand's K side, so with the row layouts each wave's V tile goes
// from HBM straight into LDS (global_load_lds) and is read back transposed
// (ds_read_b64_tr_b16); the x-split layout stores V transposed already.  Every
// wave keeps the next tile's K and V loads in flight while it computes the
// current one, and issues them only once the current tile has landed (one
// tile of loads outstanding per wave; at d = 256 with the row layouts K runs
// one more tile ahead, and the x-split layout at d = 256 keeps one tile and no
// prefetch).  Where a wave reads only one KV head's slice of each token row,
// K goes through LDS as well (KD).  K and V are read once, with non-temporal
// loads.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "gqa_decode.h"

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t uint4_t __attribute__((ext_vector_type(4)));
typedef uint32_t uint2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kTile = 32;            // tokens per wave iteration (two 16-token MFMA row blocks)
constexpr int kMaxHeadsPerGroup = 8; // waves (KV heads) per partition workgroup, at most

// Waves per partition workgroup for head dimension D.  Up to d = 128 a wave
// fits in 256 registers, two waves per SIMD; at d = 256 its two K/V tiles
// alone take 256, so a workgroup has at most 4 waves (one per SIMD) and each
// wave may use the SIMD's whole 512-entry register file (arch + acc).
__host__ __device__ constexpr int max_heads_per_group(int d) {
  return d > 128 ? 4 : kMaxHeadsPerGroup;
}
constexpr int kMaxGrid = 2048;       // persistent grid cap (two partial slots per workgroup)
constexpr int kMinChunkTiles = 2;    // smallest balanced share: 2 tiles = 64 tokens
constexpr int kWavesPerCu = 4;       // balanced grid: waves per CU it aims for (see balanced_grid)
constexpr int kMaxSeqsBalanced = 7168;   // its prefix shares LDS with two V tiles per wave
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- dtypes --

struct F16 {
  static __device__ __forceinline__ float4_t mfma(uint4_t a, uint4_t b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                  __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
  }
  // round-to-nearest-even narrowing; returns the 16 storage bits
  static __device__ __forceinline__ uint32_t narrow(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
  }
  static __device__ __forceinline__ float widen(uint32_t bits) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
  }
  // c + a.lo * b.lo + a.hi * b.hi in fp32 (v_dot2_f32_f16)
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                  false);
  }
};

struct BF16 {
  static __device__ __forceinline__ float4_t mfma(uint4_t a, uint4_t b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t narrow(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
  }
  static __device__ __forceinline__ float widen(uint32_t bits) {
    return __builtin_bit_cast(float, bits << 16);
  }
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
  }
};

// ------------------------------------------------------------ parameters --

// Division by a runtime divisor d >= 1 as a multiply and a shift, exact for
// numerators below 2^30: shift s = 30 + ceil(log2 d) and multiplier
// m = ceil(2^s / d) <= 2^31 (the round-up method of Granlund and Montgomery).
// The kernels' index arithmetic divides by sizes the host knows, and a
// hardware division is a long instruction sequence on the path to the first
// load.
struct FastDiv {
  uint32_t m;
  int s;
  __device__ __forceinline__ uint32_t div(uint32_t n) const {
    return (uint32_t)(((uint64_t)n * m) >> s);
  }
};
inline FastDiv fast_div(uint32_t d) {
  int l = 0;
  while ((uint64_t(1) << l) < d) ++l;
  return FastDiv{(uint32_t)(((uint64_t(1) << (30 + l)) + d - 1) / d), 30 + l};
}

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  const int32_t* block_table;   // paged only
  const int32_t* ctx_lens;      // paged only
  float2* part_ml;              // partial (m in log2 units, l) per (slot, query head)
  float* part_o;                // partial un-normalised O row per (slot, query head)
  int4* desc;                   // balanced mode, paged: per (sequence, head group) segment record
  int* cnt;                     // fused merge: segments finished per (sequence, head group)
  int* fixed_hdr;               // fixed mode, paged: [0] items listed
  int2* items;                  // fixed mode, paged: (s * h_kv + j0, 4 p + log2 heads), largest first
  int plan_shift;               // fixed mode, paged: size class = tiles * heads >> plan_shift
  int hpw2;                     // fixed mode, paged: KV heads per item of a split sequence
  int num_seqs;
  int h_q;
  int h_kv;
  int group;                    // G = h_q / h_kv
  int tq;                       // query tokens per sequence (T_q)
  int ncol;                     // G * T_q: query rows that share one KV head (<= 16)
  int hpw;                      // KV heads per workgroup
  int wph;                      // waves per KV head (they split each segment's tiles)
  int n_groups;                 // h_kv / hpw
  int s_kv;                     // contiguous length
  int max_blocks;               // paged table width
  int bs_shift;                 // log2(block_size)
  int max_ctx;                  // clamp for ctx_lens
  int part_size;                // fixed mode: tokens per partition
  int v1_max_ctx;               // sequences this short are never split
  int max_parts;                // fixed mode: partition slots per (sequence, query head)
  int pchunk;                   // balanced mode, contiguous: tiles per workgroup share
  FastDiv pchunk_div;           //   and division by it
  FastDiv rows_div;             // division by T_q * h_q (query rows per sequence)
  FastDiv hq_div;               // division by h_q
  FastDiv g_div;                // division by G
  FastDiv hpw_div;              // division by hpw
  float c;                      // scale * log2(e)
};

// Read-only tables (block table, context lengths) are read through the
// constant address space: they are not written while a kernel runs, and a
// wave-uniform index then becomes a scalar load instead of a vector load that
// would share the vector-memory counter with the K/V stream.
template <class T>
__device__ __forceinline__ T load_const(const T* p, int64_t i) {
  typedef const __attribute__((address_space(4))) T* const_ptr;
  return ((const_ptr)p)[i];
}

template <bool PAGED>
__device__ __forceinline__ int seq_len(const Params& a, int s) {
  if constexpr (PAGED) {
    const int L = load_const(a.ctx_lens, s);
    return min(max(L, 0), a.max_ctx);
  } else {
    return a.s_kv;
  }
}

// Cache-policy operand of global_load_lds for a non-temporal load (the nt bit).
constexpr int kAuxNontemporal = 2;

// K and V are read exactly once per call, so their loads are non-temporal:
// they do not displace the partials, tables and queries the caches hold (on
// MI355X this raises the partition kernel's read rate by about a tenth).
template <class T, bool NT>
__device__ __forceinline__ T load_stream(const uint16_t* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
  else
    return *reinterpret_cast<const T*>(p);
}

// tiles of 32 tokens a sequence occupies in the balanced work space (an empty
// sequence still occupies one, so that exactly one workgroup writes its zero row)
__device__ __forceinline__ int seq_tiles(int L) { return max(1, (L + kTile - 1) / kTile); }

// Waits until every vector-memory operation of this wave has completed
// (s_waitcnt vmcnt(0); the LDS/scalar and export counters are left alone).
// The d <= 128 token loop calls it before issuing the next tile: on MI355X a
// wave with two tiles of 16-byte loads outstanding there (up to 32 per lane)
// streams slower than one that keeps at most one tile (16) in flight, and the
// CU's other waves cover the gap.
__device__ __forceinline__ void wait_tile_loads() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0x0F70);             // vmcnt 0, expcnt 7, lgkmcnt 15 (no wait)
  __builtin_amdgcn_sched_barrier(0);
}

// Orders this wave's LDS stores before its later LDS loads (and vice versa):
// the asm is a compiler memory barrier and the wait retires the wave's
// outstanding LDS operations.  Each wave only touches its own LDS tile.
__device__ __forceinline__ void wave_lds_fence() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Device-coherent vector memory access: cache policy sc1, the bits the
// compiler gives a relaxed device-scope atomic load or store on this
// architecture.  Such a store writes through its XCD's L2 and such a load does
// not take a line that another XCD may have changed from its own L2, so data
// passed between workgroups this way needs no device-scope release or acquire
// fence (which write back or invalidate the whole L2 of the XCD), only the
// completion of the stores before the atomic that publishes them.  Raw buffer
// operations carry the 16-byte width the atomic forms lack; the resource spans
// 2 GB from a wave-uniform base.
constexpr int kAuxDeviceCoherent = 16;
constexpr int kBufferWord3 = 0x00020000;        // raw buffer, 32-bit data format
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, kBufferWord3);
}
__device__ __forceinline__ void store_coherent(__amdgpu_buffer_rsrc_t r, uint32_t byte_off,
                                               float4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(uint4_t, v), r, byte_off, 0,
                                         kAuxDeviceCoherent);
}
__device__ __forceinline__ void store_coherent(__amdgpu_buffer_rsrc_t r, uint32_t byte_off,
                                               float2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(uint2_t, v), r, byte_off, 0,
                                        kAuxDeviceCoherent);
}
__device__ __forceinline__ float4_t load_coherent4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0,
                                                                            kAuxDeviceCoherent));
}
__device__ __forceinline__ float2 load_coherent2(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0,
                                                                         kAuxDeviceCoherent));
}

// Token held in k-slot e (0..7) of lane group grp: two 16-token halves, four
// consecutive tokens each.  The same slot order feeds P^T and V^T.
__device__ __forceinline__ int slot_token(int grp, int e) {
  return (e & 4) * 4 + grp * 4 + (e & 3);
}

// Staged V tiles are row-major without padding; the 16-byte chunks of a row
// are XOR-permuted so that the transposed reads of the four lane groups
// (rows 4 grp + e) fall in distinct LDS banks.
__device__ __forceinline__ int v_swizzle(int row) { return 2 * ((row >> 2) & 3); }

template <int D>
struct Geo {
  static constexpr int KK = D / 32;        // MFMA steps over d for Q.K^T
  static constexpr int NB = D / 16;        // 16-row blocks of O^T
  static constexpr int CH = D / 8;         // 16-byte chunks per K/V row
  static constexpr int RPI = 64 / CH;      // V rows per 16-byte load instruction
  static constexpr int NIT = kTile / RPI;  // V load instructions per tile
  static constexpr int V_TILE = kTile * D; // uint16 per staged V tile
};

// With the row layouts the V tile goes from HBM straight into LDS (gfx950's
// global_load_lds_dwordx4, which writes lane l's 16 bytes at the LDS base +
// 16 l), double-buffered so that the next tile's V lands while the current
// one is read; the matrix-core operand V^T is then read back with the
// transposing LDS read ds_read_b64_tr_b16.  No V passes through registers.
// The LDS of one wave of the matrix-core segment code, in uint16, is thus its
// two V tiles (row layouts), each followed by its K tile when K also goes
// through LDS (KD), or one tile for the sub-wave state exchange (x-split).
template <int D, bool XS, bool KD = false>
__host__ __device__ constexpr int wave_lds_elems() {
  return (XS ? 1 : 2) * (KD ? 2 : 1) * Geo<D>::V_TILE;
}

// ------------------------------------------------- one wave, one segment --
//
// One wave computes the partial triple of tokens [t0, t1) of (sequence s,
// KV head j) for the G * T_q query rows of that KV head (T_q query tokens of
// G heads each, every one attending to all L_s keys) and either stores the
// normalised output (complete == true: the segment is the whole sequence) or
// the fp32 partial at pml[c * ml_stride], po[c * o_stride] for column
// c = tau * G + g.  The wave walks its 32-token tiles in order.  vt is the
// wave's LDS tile inside smem (V staging with the row layouts; the sub-wave
// state exchange with SPLIT), mlx the workgroup's (m, l) exchange (SPLIT).
// NT selects non-temporal K/V loads.
//
// XS selects the x-split paged cache (kernel-map page, "paged_attention_v1",
// the key_cache layout [num_blocks, h_kv, d / x, block_size, x] with x = 8
// elements = 16 bytes) with V as [num_blocks, h_kv, d, block_size].  A K
// load still brings 8 consecutive d of one token; a V load brings 4
// consecutive tokens of one d, which is already the transposed operand the
// P.V product needs, so V goes from HBM to the matrix core without the LDS
// tile.

// KD (row layouts, d <= 128) sends K through LDS as well: each instruction
// then reads 4 whole 256-byte head slices of token rows (the V pattern)
// instead of 64 bytes of 16 rows, and the matrix-core operand is read back
// with 16-byte LDS reads.  It pays where a workgroup reads one KV head, 256 B
// of each token row (the paged fixed decomposition's single-pass items), and
// costs a little where four waves already read 1 KB runs of each row.
//
// WT writes a partial with device-coherent stores (store_coherent) relative to
// a.part_ml / a.part_o, for a merge by another workgroup of the same launch.
template <class DT, int D, bool PAGED, bool XS, bool NT, bool SPLIT, bool KD = false,
          bool WT = false>
__device__ __forceinline__ void wave_segment(const Params& a, uint16_t* smem, uint16_t* vt,
                                             float2* mlx, int s, int j, int t0, int t1,
                                             bool complete, float2* pml,
                                             int64_t ml_stride, float* po, int64_t o_stride) {
  using Gm = Geo<D>;
  constexpr int KK = Gm::KK, NB = Gm::NB, CH = Gm::CH, RPI = Gm::RPI, NIT = Gm::NIT;
  static_assert(!KD || (!XS && D <= 128), "K through LDS: row layouts, d <= 128");
  // uniform over the wave; say so, so that addressing and branches stay scalar
  s = __builtin_amdgcn_readfirstlane(s);
  j = __builtin_amdgcn_readfirstlane(j);
  t0 = __builtin_amdgcn_readfirstlane(t0);
  t1 = __builtin_amdgcn_readfirstlane(t1);
  const int lane = threadIdx.x & 63;
  // SPLIT: the wph waves of a KV head split the segment's tiles evenly and
  // sub-wave u walks [u0, u1); tile masking then uses u1, the output logic the
  // whole segment.  (A compile-time switch: the extra scalars would push the
  // one-wave-per-head kernels past their register budget.)
  int sub = 0, w = 0;
  bool seg_empty = false;
  if constexpr (SPLIT) {
    w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    sub = (int)a.hpw_div.div(w);
    const int n_all = t1 > t0 ? (t1 - t0 + kTile - 1) / kTile : 0;
    const int u0 = t0 + kTile * (sub * n_all / a.wph);
    const int u1 = min(t1, t0 + kTile * ((sub + 1) * n_all / a.wph));
    seg_empty = t1 <= t0;
    t0 = u0;
    t1 = u1;
  }
  const int col = lane & 15;                     // head column / K row within a half
  const int grp = lane >> 4;                     // 16-lane group
  const int G = a.group;
  // column col < ncol is query token tau = col / G, query head j G + col % G
  const bool live = col < a.ncol;
  const int tau = live ? (int)a.g_div.div(col) : 0;
  const int64_t qo_row = ((int64_t)s * a.tq + tau) * a.h_q + j * G + (live ? col - tau * G : 0);

  // ---- Q^T operand: lane holds q[head col][8 d of chunk kk*4+grp]; zero rows pad G to 16
  uint4_t qop[KK];
  {
    const uint16_t* qrow = a.q + qo_row * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qop[kk] = live ? *reinterpret_cast<const uint4_t*>(qrow + 8 * (kk * 4 + grp))
                     : uint4_t{0u, 0u, 0u, 0u};
  }

  float m_run = -INFINITY;     // running max of head col, log2 units (same in all 4 groups)
  float l_run = 0.f;           // this lane's share of the running sum
  float4_t acc[NB];            // acc[nb][r] = O[head col][16 nb + 4 grp + r]
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = float4_t{0.f, 0.f, 0.f, 0.f};

  const int64_t trow = (int64_t)s * a.max_blocks;
  const uint32_t tok_stride = (uint32_t)a.h_kv * D;   // elements between consecutive tokens
  const int bs_mask = (1 << a.bs_shift) - 1;

  struct TileRows {                               // (V goes to LDS, not registers)
    uint4_t k[KD ? 1 : 2][KD ? 1 : KK];          // (KD: K goes to LDS as well)
  };
  struct TileX {
    uint4_t k[2][KK];
    uint2_t v[NB][2];                             // [d block][half]: 4 tokens of d = 16 nb + col
  };
  using Tile = std::conditional_t<XS, TileX, TileRows>;

  // Issue the global loads of the tile starting at token tb (tb < t1): all of
  // them (part 0), K only (part 1) or V only (part 2).  Each
  // 16-token half has a wave-uniform base pointer; lanes add small 32-bit
  // offsets.  Rows past t1 are clamped to the last live token of the segment,
  // so every load is in bounds and unconditional; those rows are masked
  // afterwards (score -inf, hence a zero weight on a finite V row).
  auto load = [&](Tile& T, int tb, uint16_t* vbuf, int part = 0) {
    const uint16_t* kb[2];
    const uint16_t* vb[2];
    int last[2];                                  // last live row of each half
    if constexpr (XS) {
      // Each (block, KV head) owns D * block_size contiguous elements in both
      // caches.  A half past t1 reads the 16-aligned run holding token t1 - 1
      // instead (same block, in bounds); its weights are zero and its V
      // elements are cleared in compute().
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const int th = min(tb + 16 * hb, t1 - 1);
        last[hb] = min(15, t1 - 1 - th);
        const int32_t blk = load_const(a.block_table, trow + (th >> a.bs_shift));
        const int64_t region = ((int64_t)blk * a.h_kv + j) * (D << a.bs_shift);
        kb[hb] = a.k + region + (th & bs_mask) * 8;
        vb[hb] = a.v + region + (min(tb + 16 * hb, (t1 - 1) & ~15) & bs_mask);
      }
      // per-lane offsets, computed once; the d-chunk / d-row steps are
      // wave-uniform and go to the scalar base
      const uint32_t v_lane = ((uint32_t)col << a.bs_shift) + 4 * grp;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const uint32_t k_lane = ((uint32_t)grp << (a.bs_shift + 3)) + min(col, last[hb]) * 8;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const uint16_t* kbase = kb[hb] + ((int64_t)(kk * 4) << (a.bs_shift + 3));
          T.k[hb][kk] = load_stream<uint4_t, NT>(kbase + k_lane);
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const uint16_t* vbase = vb[hb] + ((int64_t)(16 * nb) << a.bs_shift);
          T.v[nb][hb] = load_stream<uint2_t, NT>(vbase + v_lane);
        }
    } else {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const int th = min(tb + 16 * hb, t1 - 1);   // 16-aligned unless past t1
        last[hb] = min(15, t1 - 1 - th);
        int64_t base;
        if constexpr (PAGED) {
          const int32_t blk = load_const(a.block_table, trow + (th >> a.bs_shift));
          base = ((((int64_t)blk << a.bs_shift) + (th & bs_mask)) * a.h_kv + j) * D;
        } else {
          base = (((int64_t)s * a.s_kv + th) * a.h_kv + j) * D;
        }
        kb[hb] = a.k + base;
        vb[hb] = a.v + base;
      }
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        if (part == 1) break;
        const int r = it * RPI + lane / CH;
        const int hb = r >> 4;                      // uniform per instruction
        // lane l fills LDS position l % CH of row r, which holds chunk
        // (l % CH) ^ swizzle(r) of the row (the staged layout below)
        const int c = (lane % CH) ^ v_swizzle(r);
        const uint32_t off = (uint32_t)min(r & 15, last[hb]) * tok_stride + c * 8;
        __builtin_amdgcn_global_load_lds(
            reinterpret_cast<const void*>(vb[hb] + off),
            (__attribute__((address_space(3))) void*)(vbuf + it * 64 * 8), 16, 0,
            NT ? kAuxNontemporal : 0);
      }
      if constexpr (KD) {
        // the K tile after the V tile: lane l fills position l % CH of row r
        // with chunk (l % CH) ^ (r % CH), so that the 16 rows an operand read
        // touches at one chunk fall in distinct LDS banks
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
          const int r = it * RPI + lane / CH;
          const int hb = r >> 4;
          const int c = (lane % CH) ^ (r & (CH - 1));
          const uint32_t off = (uint32_t)min(r & 15, last[hb]) * tok_stride + c * 8;
          __builtin_amdgcn_global_load_lds(
              reinterpret_cast<const void*>(kb[hb] + off),
              (__attribute__((address_space(3))) void*)(vbuf + Gm::V_TILE + it * 64 * 8), 16, 0,
              NT ? kAuxNontemporal : 0);
        }
      } else if (part != 2) {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const uint32_t roff = (uint32_t)min(col, last[hb]) * tok_stride;
#pragma unroll
          for (int kk = 0; kk < KK; ++kk)
            T.k[hb][kk] = load_stream<uint4_t, NT>(kb[hb] + roff + 8 * (kk * 4 + grp));
        }
      }
    }
  };

  // fold the tile starting at token tb into (m_run, l_run, acc)
  auto compute = [&](const Tile& T, int tb, const uint16_t* vbuf) {
    // scores S^T = K . Q^T
    float4_t sc[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      sc[hb] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        uint4_t kop;
        if constexpr (KD) {
          const int row = 16 * hb + col;
          const int pos = (kk * 4 + grp) ^ (row & (CH - 1));
          kop = *reinterpret_cast<const uint4_t*>(vbuf + Gm::V_TILE + row * D + pos * 8);
        } else {
          kop = T.k[hb][kk];
        }
        sc[hb] = DT::mfma(kop, qop[kk], sc[hb]);
      }
    }
    // online softmax (base 2); the lane holds tokens slot_token(grp, e) of head col
    float x[8];
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int tok = tb + slot_token(grp, e);
      x[e] = tok < t1 ? sc[e >> 2][e & 3] * a.c : -INFINITY;
      mx = fmaxf(mx, x[e]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);          // finite: the tile holds a live token
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    // P as a hi + lo pair in the storage dtype (about twice its significand)
    uint32_t phi[4], plo[4];
    float psum = 0.f;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      uint32_t h2 = 0, l2 = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float pe = __builtin_amdgcn_exp2f(x[2 * e2 + h] - m_new);
        psum += pe;
        const uint32_t hi = DT::narrow(pe);
        const uint32_t lo = DT::narrow(pe - DT::widen(hi));
        h2 |= hi << (16 * h);
        l2 |= lo << (16 * h);
      }
      phi[e2] = h2;
      plo[e2] = l2;
    }
    l_run = l_run * alpha + psum;
    const uint4_t phi4{phi[0], phi[1], phi[2], phi[3]};
    const uint4_t plo4{plo[0], plo[1], plo[2], plo[3]};
    if constexpr (XS) {
      // O^T += V^T . P^T with V^T straight from the loads; in a tile that
      // reaches past t1, V elements of tokens >= t1 (possibly NaN) are cleared
      uint2_t keep[2] = {uint2_t{~0u, ~0u}, uint2_t{~0u, ~0u}};
      if (tb + kTile > t1) {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const int kc = t1 - (tb + 16 * hb + 4 * grp);   // live tokens of the lane's run
          keep[hb].x = (kc >= 1 ? 0x0000FFFFu : 0u) | (kc >= 2 ? 0xFFFF0000u : 0u);
          keep[hb].y = (kc >= 3 ? 0x0000FFFFu : 0u) | (kc >= 4 ? 0xFFFF0000u : 0u);
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint4_t vop{T.v[nb][0].x & keep[0].x, T.v[nb][0].y & keep[0].y,
                          T.v[nb][1].x & keep[1].x, T.v[nb][1].y & keep[1].y};
        acc[nb] *= alpha;
        acc[nb] = DT::mfma(vop, phi4, acc[nb]);
        acc[nb] = DT::mfma(vop, plo4, acc[nb]);
      }
    } else {
      // O^T += V^T . P^T, V^T read transposed from the staged tile
      wave_lds_fence();
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        // ds_read_b64_tr_b16: within each 16-lane group, lane i receives
        // element i % 4 of the 8-byte loads of lanes 4 e + i / 4 (e = 0..3).
        // Lane (col, grp) loads row slot_token(grp, col / 4) (then the same
        // token + 16) at d = 16 nb + 4 (col % 4), so it receives
        // V[slot_token(grp, e)][16 nb + col]: its V^T operand row.
        const int d0 = 16 * nb + 4 * (col & 3);
        const int r0 = slot_token(grp, col >> 2), r1 = r0 + 16;
        typedef short short4_t __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) short4_t lds_short4_t;
        const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(
            const_cast<uint16_t*>(vbuf) + r0 * D + (((d0 >> 3) ^ v_swizzle(r0)) << 3) + (d0 & 7)));
        const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(
            const_cast<uint16_t*>(vbuf) + r1 * D + (((d0 >> 3) ^ v_swizzle(r1)) << 3) + (d0 & 7)));
        const uint2_t l2 = __builtin_bit_cast(uint2_t, lo), h2 = __builtin_bit_cast(uint2_t, hi);
        const uint4_t vop{l2.x, l2.y, h2.x, h2.y};
        acc[nb] *= alpha;
        acc[nb] = DT::mfma(vop, phi4, acc[nb]);
        acc[nb] = DT::mfma(vop, plo4, acc[nb]);
      }
      wave_lds_fence();                               // reads retire before the next stores
    }
  };

  // ---- token loop: two register tiles ping-ponged so that the next tile's
  //      loads are in flight while the current one is computed.  The steady
  //      state issues its loads unconditionally and the last one or two tiles
  //      are peeled, so every wait count the compiler derives is static; the
  //      scheduling barriers keep each prefetch ahead of the compute it
  //      overlaps.  The current tile has landed before the next one is issued,
  //      so a wave never has more than one tile of loads outstanding (at
  //      d = 256 with the row layouts, one tile plus the K half of the next).
  int n = t1 > t0 ? (t1 - t0 + kTile - 1) / kTile : 0;
  // V buffers (row layouts): tile A stages into vt and tile B into the wave's
  // second tile (with KD each V tile is followed by its K tile); the x-split
  // layout stages nothing
  uint16_t* const vbA = vt;
  uint16_t* const vbB = XS ? vt : vt + (KD ? 2 : 1) * Geo<D>::V_TILE;
  if constexpr (D > 128 && XS) {
    // d = 256, x-split: V goes to registers, so one register tile (32 KB of
    // K/V per wave).  A wave waits for each tile; the other waves of the CU
    // keep 3 x 32 KB in flight meanwhile.
    Tile A;
    for (int tb = t0; n > 0; --n, tb += kTile) {
      load(A, tb, vbA);
      compute(A, tb, vbA);
    }
  } else if (D > 128 && n > 0) {
    // d = 256: K one tile further ahead than V, in three register tiles (V
    // keeps its two LDS tiles, all the LDS four such waves can have).  Before
    // tile t is computed, V(t+1) and K(t+2) are issued, and the wait for tile t
    // lets K(t+1), issued after V(t), stay in flight.  Same box, us per
    // partition launch on 2 sequences of 32768 tokens, 32/8 heads: 83.4 ->
    // 81.9; at d = 128 the same order was 1-3% slower.
    constexpr int NK = 2 * KK;                    // K load instructions per tile
    Tile T0, T1, T2;
    auto body = [&](Tile& Tc, Tile& Tn2, uint16_t* vc, uint16_t* vn, int t) {
      const int tb = t0 + t * kTile;
      __builtin_amdgcn_sched_barrier(0);
      if (t + 1 < n)
        __builtin_amdgcn_s_waitcnt((NK & 15) | ((NK >> 4) << 14) | 0x0F70);   // vmcnt(NK)
      else
        __builtin_amdgcn_s_waitcnt(0x0F70);                                    // vmcnt(0)
      __builtin_amdgcn_sched_barrier(0);
      if (t + 1 < n) load(Tn2, tb + kTile, vn, 2);          // V(t+1)
      if (t + 2 < n) load(Tn2, tb + 2 * kTile, vn, 1);      // K(t+2)
      __builtin_amdgcn_sched_barrier(0);
      compute(Tc, tb, vc);
    };
    load(T0, t0, vbA);
    if (n > 1) load(T1, t0 + kTile, vbB, 1);
    for (int t = 0; t < n; t += 6) {              // K tile t % 3, V tile t % 2
      body(T0, T2, vbA, vbB, t);
      if (t + 1 < n) body(T1, T0, vbB, vbA, t + 1);
      if (t + 2 < n) body(T2, T1, vbA, vbB, t + 2);
      if (t + 3 < n) body(T0, T2, vbB, vbA, t + 3);
      if (t + 4 < n) body(T1, T0, vbA, vbB, t + 4);
      if (t + 5 < n) body(T2, T1, vbB, vbA, t + 5);
    }
  } else if (n > 0) {
    Tile A, B;
    int tb = t0;
    load(A, tb, vbA);
    while (n >= 3) {
      wait_tile_loads();
      load(B, tb + kTile, vbB);
      __builtin_amdgcn_sched_barrier(0);
      compute(A, tb, vbA);
      wait_tile_loads();
      load(A, tb + 2 * kTile, vbA);
      __builtin_amdgcn_sched_barrier(0);
      compute(B, tb + kTile, vbB);
      tb += 2 * kTile;
      n -= 2;
    }
    // (the LDS-staged V of the last tiles has landed only after a wait: the
    // compiler tracks register operands, not the LDS the loads write)
    if (n == 2) {
      wait_tile_loads();
      load(B, tb + kTile, vbB);
      __builtin_amdgcn_sched_barrier(0);
      compute(A, tb, vbA);
      wait_tile_loads();
      compute(B, tb + kTile, vbB);
    } else {
      wait_tile_loads();
      compute(A, tb, vbA);
    }
  }

  // ---- epilogue: each lane owns head col, d = 16 nb + 4 grp + r
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if constexpr (SPLIT) {
    // Merge the wph sub-wave states of this KV head ("_merge_running" in sub-wave
    // order, an empty share (-inf, 0, 0) weighing 0) into sub-wave 0, through
    // LDS: each wave parks its accumulators in its own tile region (64 D bytes,
    // the size of a V tile) and its (m, l) per column in mlx.  Every wave of the
    // workgroup walks the same segments, so the barriers are uniform.
    float4_t* park = reinterpret_cast<float4_t*>(vt);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) park[nb * 64 + lane] = acc[nb];
    if (grp == 0) mlx[w * 16 + col] = make_float2(m_run, l_run);
    __syncthreads();
    if (sub == 0) {
      for (int u = 1; u < a.wph; ++u) {
        const int w2 = w + u * a.hpw;
        const float2 o2 = mlx[w2 * 16 + col];
        const float m_new = fmaxf(m_run, o2.x);
        const float a1 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
        const float a2 = o2.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(o2.x - m_new);
        const float4_t* other =
            reinterpret_cast<const float4_t*>(smem + w2 * wave_lds_elems<D, XS, KD>());
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = acc[nb] * a1 + other[nb * 64 + lane] * a2;
        l_run = l_run * a1 + o2.y * a2;
        m_run = m_new;
      }
    }
    __syncthreads();                              // parked states read before the next segment
    if (sub != 0) return;
  }
  if (!live) return;
  if (complete) {
    uint16_t* dst = a.out + qo_row * D + 4 * grp;
    if constexpr (!SPLIT) seg_empty = t1 <= t0;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      uint32_t w01, w23;
      if (seg_empty) {
        w01 = w23 = 0u;
      } else {
        w01 = DT::narrow(acc[nb][0] / l_run) | (DT::narrow(acc[nb][1] / l_run) << 16);
        w23 = DT::narrow(acc[nb][2] / l_run) | (DT::narrow(acc[nb][3] / l_run) << 16);
      }
      *reinterpret_cast<uint2*>(dst + 16 * nb) = make_uint2(w01, w23);
    }
  } else if constexpr (WT) {
    const uint32_t o0 = (uint32_t)((po - a.part_o) + (int64_t)col * o_stride + 4 * grp) * 4;
    const __amdgpu_buffer_rsrc_t ro = coherent_rsrc(a.part_o);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) store_coherent(ro, o0 + 64 * nb, acc[nb]);
    if (grp == 0)
      store_coherent(coherent_rsrc(a.part_ml),
                     (uint32_t)((pml - a.part_ml) + (int64_t)col * ml_stride) * 8,
                     make_float2(m_run, l_run));
  } else {
    float* dst = po + (int64_t)col * o_stride + 4 * grp;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) *reinterpret_cast<float4_t*>(dst + 16 * nb) = acc[nb];
    if (grp == 0) pml[(int64_t)col * ml_stride] = make_float2(m_run, l_run);
  }
}

// ------------------------------------ one wave, one segment, vector ALU --
//
// The partial triple of wave_segment with both products on the vector ALU
// instead of the matrix cores: packed two-element dot products with fp32
// accumulation (v_dot2_f32_f16 / v_dot2_f32_bf16).  It is there to compare
// the two units on identical loads (the tile, its lane layout and the
// non-temporal loads of the row layouts), for d = 128 and NC = 4 or 8
// columns (G * T_q <= NC; zero query rows pad the rest).
//   scores   lane (col, grp) holds K rows 16 hb + col, d chunks 4 kk + grp,
//            and forms partial dot products with every query row (the wave
//            parks them in LDS; a read is a broadcast to the 16 lanes of a
//            row).  Two swap-and-add steps across rows (v_permlane16_swap,
//            v_permlane32_swap) complete them and leave the lane the scores
//            of token 16 (grp >> 1) + col for columns NH (grp & 1) + h',
//            h' < NH = NC / 2.
//   softmax  tile maxima over the 32 lanes of a column set, then exchanged,
//            so that every lane keeps m of all NC columns; P, as the hi + lo
//            pair of wave_segment, goes to LDS.
//   P.V      V is staged in LDS as in wave_segment.  Lane (col, grp) owns
//            O[h][8 col + e] of the columns h = 4 i + grp, i < NC / 4, over
//            all tokens: it reads rows 2k and 2k + 1 of d chunk col, repacks
//            them into token-pair halves, and one dot2 folds both tokens of a
//            pair into one output element.

constexpr int kDot2D = 128;                       // head dimension of the vector-ALU variant

// LDS per wave, in uint16: the query rows [NC][D], the V tile [32][D], P hi and lo [2][NC][32]
__host__ __device__ constexpr int dot2_wave_elems(int nc) {
  return nc * kDot2D + kTile * kDot2D + 2 * nc * kTile;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xF, 0xF, false));
}

// Reductions over the 16 lanes of a row; every lane receives the result.
// quad_perm [1,0,3,2] and [2,3,0,1], then row_half_mirror and row_mirror
// (after each step the lanes being combined hold equal partial results).
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  return fmaxf(x, dpp<0x140>(x));
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  return x + dpp<0x140>(x);
}

// v_permlane16_swap: the odd 16-lane rows of a trade places with the even
// rows of b, so a = [a0, b0, a2, b2], b = [a1, b1, a3, b3] afterwards.
// v_permlane32_swap: the upper 32 lanes of a trade places with the lower 32
// of b, so a = [a_lo, b_lo], b = [a_hi, b_hi] afterwards.
// Written as asm with both operands read and written: the compiler's builtins
// for these instructions (ROCm 7.2) return the first operand's new value as
// both results.  The two wait states cover a VALU write of an operand just
// before the swap, as the compiler itself inserts them.
__device__ __forceinline__ void swap_rows16(float& a, float& b) {
  __asm__("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap_halves32(float& a, float& b) {
  __asm__("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

__device__ __forceinline__ float pick4(const float* v, int g) {
  return g == 0 ? v[0] : g == 1 ? v[1] : g == 2 ? v[2] : v[3];
}

template <class DT, bool PAGED, int NC>
__device__ __forceinline__ void wave_segment_dot2(const Params& a, uint16_t* vt, int s, int j,
                                                  int t0, int t1, bool complete, float2* pml,
                                                  int64_t ml_stride, float* po, int64_t o_stride) {
  constexpr int D = kDot2D;
  using Gm = Geo<D>;
  constexpr int KK = Gm::KK, CH = Gm::CH, RPI = Gm::RPI, NIT = Gm::NIT;
  constexpr int NH = NC / 2;                      // score columns per lane
  constexpr int NO = NC / 4;                      // output columns per lane
  static_assert(RPI == 4 && CH == 16 && (NC == 4 || NC == 8), "vector-ALU tile geometry");
  s = __builtin_amdgcn_readfirstlane(s);
  j = __builtin_amdgcn_readfirstlane(j);
  t0 = __builtin_amdgcn_readfirstlane(t0);
  t1 = __builtin_amdgcn_readfirstlane(t1);
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const bool odd = grp & 1;
  const int G = a.group;
  uint32_t* const qs = reinterpret_cast<uint32_t*>(vt);   // query rows, half pairs [NC][D / 2]
  uint16_t* const vs = vt + NC * D;                        // V tile [kTile][D]
  uint16_t* const ps16 = vs + kTile * D;                   // P: hi [NC][kTile], then lo
  const uint32_t* const ps = reinterpret_cast<const uint32_t*>(ps16);   // token pairs

  // ---- park the query rows in LDS; rows past ncol are zero
  wave_lds_fence();                               // the previous segment's reads come first
#pragma unroll
  for (int i = 0; i < NC / RPI; ++i) {
    const int h = i * RPI + grp;
    uint4_t v{0u, 0u, 0u, 0u};
    if (h < a.ncol) {
      const int tau = (int)a.g_div.div(h);
      const int64_t row = ((int64_t)s * a.tq + tau) * a.h_q + j * G + (h - tau * G);
      v = *reinterpret_cast<const uint4_t*>(a.q + row * D + 8 * col);
    }
    *reinterpret_cast<uint4_t*>(qs + h * (D / 2) + 4 * col) = v;
  }
  wave_lds_fence();

  float m_run[NC];                                // running max per column, log2 units (all lanes)
  float l_run[NH];                                // this lane's share of its score columns' sums
  float acc[NO][8];                               // O[4 i + grp][8 col + e]
#pragma unroll
  for (int h = 0; h < NC; ++h) m_run[h] = -INFINITY;
#pragma unroll
  for (int h = 0; h < NH; ++h) l_run[h] = 0.f;
#pragma unroll
  for (int i = 0; i < NO; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;

  const int64_t trow = (int64_t)s * a.max_blocks;
  const uint32_t tok_stride = (uint32_t)a.h_kv * D;
  const int bs_mask = (1 << a.bs_shift) - 1;

  struct Tile {
    uint4_t k[2][KK];
    uint4_t v[NIT];
  };
  // the row-layout loads of wave_segment: rows past t1 read the last live row
  auto load = [&](Tile& T, int tb) {
    const uint16_t* kb[2];
    const uint16_t* vb[2];
    int last[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int th = min(tb + 16 * hb, t1 - 1);
      last[hb] = min(15, t1 - 1 - th);
      int64_t base;
      if constexpr (PAGED) {
        const int32_t blk = load_const(a.block_table, trow + (th >> a.bs_shift));
        base = ((((int64_t)blk << a.bs_shift) + (th & bs_mask)) * a.h_kv + j) * D;
      } else {
        base = (((int64_t)s * a.s_kv + th) * a.h_kv + j) * D;
      }
      kb[hb] = a.k + base;
      vb[hb] = a.v + base;
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int r = it * RPI + grp;
      const int hb = r >> 4;
      const uint32_t off = (uint32_t)min(r & 15, last[hb]) * tok_stride + 8 * col;
      T.v[it] = load_stream<uint4_t, true>(vb[hb] + off);
    }
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const uint32_t roff = (uint32_t)min(col, last[hb]) * tok_stride;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        T.k[hb][kk] = load_stream<uint4_t, true>(kb[hb] + roff + 8 * (kk * 4 + grp));
    }
  };

  const int tt = 16 * (grp >> 1) + col;           // the lane's token within a tile (scores)

  auto compute = [&](const Tile& T, int tb) {
    // stage V: row 4 it + grp, d chunk col
#pragma unroll
    for (int it = 0; it < NIT; ++it)
      *reinterpret_cast<uint4_t*>(vs + (it * RPI + grp) * D + 8 * col) = T.v[it];
    // ---- scores: partial sums over the lane's d chunks, then across the four rows
    float sc[2][NC];
#pragma unroll
    for (int h = 0; h < NC; ++h) sc[0][h] = sc[1][h] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int h = 0; h < NC; ++h) {
        const uint4_t qv = *reinterpret_cast<const uint4_t*>(qs + h * (D / 2) + (4 * kk + grp) * 4);
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int e = 0; e < 4; ++e) sc[hb][h] = DT::dot2(T.k[hb][kk][e], qv[e], sc[hb][h]);
      }
    float x[NH];
    float alpha[NC];
    {
      float m_tile[NC];
      const bool live = tb + tt < t1;
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        float a0 = sc[0][h], b0 = sc[0][h + NH], a1 = sc[1][h], b1 = sc[1][h + NH];
        swap_rows16(a0, b0);
        swap_rows16(a1, b1);
        float x0 = a0 + b0, x1 = a1 + b1;         // even rows: column h; odd rows: h + NH
        swap_halves32(x0, x1);
        x[h] = live ? (x0 + x1) * a.c : -INFINITY;
        float mx = row_max16(x[h]);
        float my = mx;
        swap_halves32(mx, my);
        mx = fmaxf(mx, my);                       // tile max of the lane's column
        float ma = mx, mb = mx;
        swap_rows16(ma, mb);                      // ma: column h, mb: column h + NH
        m_tile[h] = ma;
        m_tile[h + NH] = mb;
      }
#pragma unroll
      for (int h = 0; h < NC; ++h) {
        const float m_new = fmaxf(m_run[h], m_tile[h]);   // finite: the tile holds a live token
        alpha[h] = __builtin_amdgcn_exp2f(m_run[h] - m_new);
        m_run[h] = m_new;
      }
    }
    // ---- P (hi + lo pair in the storage dtype) to LDS
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const float mh = odd ? m_run[h + NH] : m_run[h];
      const float ah = odd ? alpha[h + NH] : alpha[h];
      const float p = __builtin_amdgcn_exp2f(x[h] - mh);
      l_run[h] = l_run[h] * ah + p;
      const uint32_t hi = DT::narrow(p);
      const uint32_t lo = DT::narrow(p - DT::widen(hi));
      uint16_t* dst = ps16 + (h + (odd ? NH : 0)) * kTile + tt;
      dst[0] = (uint16_t)hi;
      dst[NC * kTile] = (uint16_t)lo;
    }
    wave_lds_fence();
    // ---- O += P . V over token pairs (2k, 2k + 1), d = 8 col + e, columns 4 i + grp
#pragma unroll
    for (int i = 0; i < NO; ++i) {
      const float al = pick4(alpha + 4 * i, grp);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[i][e] *= al;
    }
    // (a rolled loop: unrolled, the LDS reads of all 16 pairs are hoisted and spill)
#pragma nounroll
    for (int q4 = 0; q4 < kTile / 8; ++q4) {      // pairs 4 q4 .. 4 q4 + 3
      uint4_t ph[NO], pl[NO];
#pragma unroll
      for (int i = 0; i < NO; ++i) {
        const int h = 4 * i + grp;
        ph[i] = *reinterpret_cast<const uint4_t*>(ps + h * (kTile / 2) + 4 * q4);
        pl[i] = *reinterpret_cast<const uint4_t*>(ps + (NC + h) * (kTile / 2) + 4 * q4);
      }
#pragma unroll
      for (int kp = 0; kp < 4; ++kp) {
        const int t = 8 * q4 + 2 * kp;
        const uint4_t r0 = *reinterpret_cast<const uint4_t*>(vs + t * D + 8 * col);
        const uint4_t r1 = *reinterpret_cast<const uint4_t*>(vs + (t + 1) * D + 8 * col);
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const uint32_t v_lo = __builtin_amdgcn_perm(r1[e2], r0[e2], 0x05040100u);  // d = 8 col + 2 e2
          const uint32_t v_hi = __builtin_amdgcn_perm(r1[e2], r0[e2], 0x07060302u);  // d + 1
#pragma unroll
          for (int i = 0; i < NO; ++i) {
            acc[i][2 * e2] = DT::dot2(v_lo, ph[i][kp], acc[i][2 * e2]);
            acc[i][2 * e2] = DT::dot2(v_lo, pl[i][kp], acc[i][2 * e2]);
            acc[i][2 * e2 + 1] = DT::dot2(v_hi, ph[i][kp], acc[i][2 * e2 + 1]);
            acc[i][2 * e2 + 1] = DT::dot2(v_hi, pl[i][kp], acc[i][2 * e2 + 1]);
          }
        }
      }
    }
    wave_lds_fence();                             // reads retire before the next tile's stores
  };

  // ---- token loop: the two-tile ping-pong of wave_segment
  int n = t1 > t0 ? (t1 - t0 + kTile - 1) / kTile : 0;
  if (n > 0) {
    Tile A, B;
    int tb = t0;
    load(A, tb);
    while (n >= 3) {
      load(B, tb + kTile);
      __builtin_amdgcn_sched_barrier(0);
      compute(A, tb);
      load(A, tb + 2 * kTile);
      __builtin_amdgcn_sched_barrier(0);
      compute(B, tb + kTile);
      tb += 2 * kTile;
      n -= 2;
    }
    if (n == 2) {
      load(B, tb + kTile);
      __builtin_amdgcn_sched_barrier(0);
      compute(A, tb);
      compute(B, tb + kTile);
    } else {
      compute(A, tb);
    }
  }

  // ---- epilogue: l of every column (its 32 lanes hold the shares)
  float l_all[NC];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    float l = row_sum16(l_run[h]);
    float l2 = l;
    swap_halves32(l, l2);
    l += l2;
    float la = l, lb = l;
    swap_rows16(la, lb);
    l_all[h] = la;
    l_all[h + NH] = lb;
  }
  const float (&o)[NO][8] = acc;
  const bool seg_empty = t1 <= t0;
#pragma unroll
  for (int i = 0; i < NO; ++i) {
    const int h = 4 * i + grp;
    if (h >= a.ncol) continue;
    const float lh = pick4(l_all + 4 * i, grp);
    if (complete) {
      const int tau = (int)a.g_div.div(h);
      const int64_t row = ((int64_t)s * a.tq + tau) * a.h_q + j * G + (h - tau * G);
      uint4_t w{0u, 0u, 0u, 0u};
      if (!seg_empty) {
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2)
          w[e2] = DT::narrow(o[i][2 * e2] / lh) | (DT::narrow(o[i][2 * e2 + 1] / lh) << 16);
      }
      *reinterpret_cast<uint4_t*>(a.out + row * D + 8 * col) = w;
    } else {
      float4_t* dst = reinterpret_cast<float4_t*>(po + (int64_t)h * o_stride + 8 * col);
      dst[0] = float4_t{o[i][0], o[i][1], o[i][2], o[i][3]};
      dst[1] = float4_t{o[i][4], o[i][5], o[i][6], o[i][7]};
      if (col == 0) pml[(int64_t)h * ml_stride] = make_float2(pick4(m_run + 4 * i, grp), lh);
    }
  }
}

// ------------------------------------------- fixed-partition decomposition --
//
// The kernel-map page's decomposition: a sequence of at most v1_max_ctx
// tokens is one partition written directly ("paged_attention_v1"); a longer
// one is cut into ceil(L / part_size) partitions whose partials land at
// [s, i, p] ("paged_attention_v2").  A work item is one partition of a group
// of KV heads.
//
// Contiguous cache: every sequence has the same length, so the items are
// equal and the host knows their number; one workgroup per item.
//
// Paged cache: the planner kernel (one workgroup) lists the items in the
// workspace largest first, by a counting sort over their size (tokens times
// heads; each thread writes the items of its sequences), and the partition
// kernel takes item b, b + grid, ... in list order
// (a grid of at most kFixedGridCap workgroups, no larger than the items can
// be), so the hardware dispatcher starts the longest items first and hands
// each CU the next item as it frees up.  Single-pass items take the host's
// head group (narrow, so that they are many and balance well); partitions of
// split sequences take groups of up to four heads (wide: a partition is
// short).  A workgroup has four waves; the waves of an item's head split its
// tiles and merge in LDS (as in the balanced kernel), so a single-pass item
// stays single-pass.  Which workgroup computes an item changes nothing in its
// result.

constexpr int kPlanBuckets = 256;                 // size classes of the planner's sort
constexpr int kPlanThreads = 1024;

// Items of a sequence of L tokens: partitions, heads per item, and size class
// (bucket 0 holds the largest items).
__device__ __forceinline__ void fixed_items(const Params& a, int L, int* n_part, int* heads,
                                            int* bucket) {
  const bool split = L > a.v1_max_ctx;
  *n_part = split ? (L + a.part_size - 1) / a.part_size : 1;
  *heads = split ? a.hpw2 : a.hpw;
  const int tiles = split ? (a.part_size + kTile - 1) / kTile : (L + kTile - 1) / kTile;
  *bucket = (kPlanBuckets - 1) - min(kPlanBuckets - 1, (tiles * *heads) >> a.plan_shift);
}

__device__ __forceinline__ int log2_heads(int h) { return h >= 4 ? 2 : h >= 2 ? 1 : 0; }

__global__ __launch_bounds__(kPlanThreads) void fixed_plan_kernel(Params a) {
  __shared__ int start[kPlanBuckets];             // items before bucket b (after the scan)
  __shared__ int fill[kPlanBuckets];              // items placed in bucket b so far
  __shared__ int wave_sum[kPlanBuckets / 64];
  for (int b = threadIdx.x; b < kPlanBuckets; b += blockDim.x) start[b] = fill[b] = 0;
  __syncthreads();
  for (int s = threadIdx.x; s < a.num_seqs; s += blockDim.x) {
    int np, nh, b;
    fixed_items(a, seq_len<true>(a, s), &np, &nh, &b);
    atomicAdd(&start[b], np * (a.h_kv / nh));
  }
  __syncthreads();
  // exclusive scan of the bucket counts: a shuffle scan per wave of 64 buckets
  const int lane = threadIdx.x & 63;
  int v = 0, incl = 0;
  if (threadIdx.x < kPlanBuckets) {
    v = incl = start[threadIdx.x];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off);
      if (lane >= off) incl += t;
    }
    if (lane == 63) wave_sum[threadIdx.x >> 6] = incl;
  }
  __syncthreads();
  if (threadIdx.x < kPlanBuckets) {
    int before = 0;
    for (int u = 0; u < (int)(threadIdx.x >> 6); ++u) before += wave_sum[u];
    start[threadIdx.x] = before + incl - v;
    if (threadIdx.x == kPlanBuckets - 1) a.fixed_hdr[0] = before + incl;   // items listed
  }
  __syncthreads();
  // item (s * h_kv + first KV head, 4 p + log2 heads)
  for (int s = threadIdx.x; s < a.num_seqs; s += blockDim.x) {
    int np, nh, b;
    fixed_items(a, seq_len<true>(a, s), &np, &nh, &b);
    const int ng = a.h_kv / nh;
    int at = start[b] + atomicAdd(&fill[b], np * ng);
    for (int p = 0; p < np; ++p)
      for (int g = 0; g < ng; ++g)
        a.items[at++] = make_int2(s * a.h_kv + g * nh, 4 * p + log2_heads(nh));
  }
}

// One item: partition p of sequence s for KV head j (this wave's head).
template <class DT, int D, bool PAGED, bool XS, bool NT, bool SPLIT, bool KD = false>
__device__ __forceinline__ void fixed_item(const Params& b, uint16_t* smem, float2* mlx, int w,
                                           int s, int j, int p) {
  const int L = seq_len<PAGED>(b, s);
  const bool split = L > b.v1_max_ctx;
  const int t0 = split ? p * b.part_size : 0;
  const int t1 = split ? min(t0 + b.part_size, L) : L;
  const int64_t row0 = ((int64_t)s * b.h_kv + j) * b.ncol;   // partial rows per (s, j, column)
  wave_segment<DT, D, PAGED, XS, NT, SPLIT, KD>(
      b, smem, smem + ((XS && !SPLIT) ? 0 : w * wave_lds_elems<D, XS, KD>()), mlx, s, j, t0, t1, !split,
      b.part_ml + row0 * b.max_parts + p, b.max_parts, b.part_o + (row0 * b.max_parts + p) * D,
      (int64_t)b.max_parts * D);
}

// Contiguous cache: one workgroup per item.  NT selects non-temporal K/V
// loads: they raise the read rate when many workgroups stream at once, but a
// lone wave that walks a whole long sequence is latency-bound and runs faster
// with ordinary loads (the host decides).  SPLIT: a group of one or two KV
// heads gives each head several waves, which split the item's tiles.
template <class DT, int D, bool XS, bool NT, bool SPLIT>
__global__ __launch_bounds__(max_heads_per_group(D) * 64) void partition_fixed_kernel(Params a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];   // V tiles per wave
  __shared__ float2 mlx[SPLIT ? kMaxHeadsPerGroup * 16 : 1];         // sub-wave (m, l) exchange
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int p = blockIdx.x % a.max_parts;
  const int rest = blockIdx.x / a.max_parts;
  const int hg = rest % a.n_groups;
  const int s = rest / a.n_groups;
  const int wj = SPLIT ? w - (int)a.hpw_div.div(w) * a.hpw : w;   // the wave's head in the group
  fixed_item<DT, D, false, XS, NT, SPLIT>(a, smem, mlx, w, s, hg * a.hpw + wj, p);
}

// Paged cache: items blockIdx.x, blockIdx.x + grid, ... of the planner's list.
// A workgroup has kFixedPagedWaves waves and runs alone on its CU: its LDS
// request is at least kFixedPagedLds, more than half of the CU's 160 KB.  On
// MI355X four waves per CU, each with one tile of loads in flight, stream
// faster than eight.  The waves of an item's head split its tiles and merge in
// LDS.
constexpr int kFixedPagedWaves = 4;
constexpr size_t kFixedPagedLds = 96 * 1024;
// K through LDS as well (wave_segment's KD): single-pass items read one KV head
// of each token row.  Same box, pages' policy, us per step: paged_b64 197.3 ->
// 177.6, mixed_b256 342.5 -> 320.4.
__host__ __device__ constexpr bool fixed_paged_kd(int d, bool xs) { return !xs && d <= 128; }

template <class DT, int D, bool XS>
__global__ __launch_bounds__(kFixedPagedWaves * 64) void partition_fixed_paged_kernel(Params a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];   // V and K tiles per wave
  __shared__ float2 mlx[kFixedPagedWaves * 16];                      // sub-wave (m, l) exchange
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_items = a.fixed_hdr[0];
  for (int idx = blockIdx.x; idx < n_items; idx += gridDim.x) {
    const int2 it = a.items[idx];
    const int s = __builtin_amdgcn_readfirstlane(it.x) / a.h_kv;
    const int j0 = __builtin_amdgcn_readfirstlane(it.x) - s * a.h_kv;
    const int code = __builtin_amdgcn_readfirstlane(it.y);
    Params b = a;
    b.hpw = 1 << (code & 3);                       // heads of this item
    b.hpw_div = FastDiv{1u << 30, 30 + (code & 3)};   // (fast_div of a power of two)
    b.wph = kFixedPagedWaves >> (code & 3);        // waves per head
    fixed_item<DT, D, true, XS, true, true, fixed_paged_kd(D, XS)>(b, smem, mlx, w, s,
                                                                  j0 + w % b.hpw, code >> 2);
  }
}

// --------------------------------------------------------- fused merge --
//
// The workgroup that finished a split range last merges it (policy flag
// GQA_POLICY_FUSED_MERGE): the n-ary "_merge_running" of the decode-long page
// over the range's n segments, in segment order, then "Final normalise +
// store".  One 16-lane slot per partial row (a query row of the head group);
// lane r holds d elements [r*D/16, (r+1)*D/16).  Partial k of the range sits
// in slot `first` (k = 0) or 2 (wg0 + k), as the balanced kernel wrote it with
// device-coherent stores; it is read back with device-coherent loads, U
// partials in flight per lane.

template <class DT, int D>
__device__ __forceinline__ void fused_range_merge(const Params& a, int s, int hg, int wg0, int n,
                                                  int first) {
  constexpr int E = D / 16;
  constexpr int U = D <= 128 ? 16 : 8;
  const __amdgpu_buffer_rsrc_t rml = coherent_rsrc(a.part_ml), ro = coherent_rsrc(a.part_o);
  const int heads = a.hpw * a.ncol;               // partial rows per slot
  const int nslot = blockDim.x / 16;
  const int r = threadIdx.x % 16;
  for (int row = threadIdx.x / 16; row < heads; row += nslot) {
    float m = -INFINITY, l = 0.f;
    float o[E];
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = 0.f;
    for (int k0 = 0; k0 < n; k0 += U) {
      float2 t2[U];
      float4_t v[U][E / 4];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (k0 + u < n) {
          const int k = k0 + u;
          const uint32_t rw = (uint32_t)((k == 0 ? first : 2 * (wg0 + k)) * heads + row);
          t2[u] = load_coherent2(rml, rw * 8);
#pragma unroll
          for (int e4 = 0; e4 < E / 4; ++e4) v[u][e4] = load_coherent4(ro, (rw * D + r * E + 4 * e4) * 4);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (k0 + u < n) {
          const float m_new = fmaxf(m, t2[u].x);  // finite: a partial holds at least one token
          const float a_old = __builtin_amdgcn_exp2f(m - m_new);
          const float a_new = __builtin_amdgcn_exp2f(t2[u].x - m_new);
          l = l * a_old + t2[u].y * a_new;
#pragma unroll
          for (int e4 = 0; e4 < E / 4; ++e4)
#pragma unroll
            for (int c = 0; c < 4; ++c)
              o[4 * e4 + c] = o[4 * e4 + c] * a_old + v[u][e4][c] * a_new;
          m = m_new;
        }
      }
    }
    // partial row -> output row: KV head j = hg * hpw + row / ncol, column c = tau * G + g
    const int c = row % a.ncol;
    const int j = hg * a.hpw + row / a.ncol;
    const int tau = (int)a.g_div.div(c);
    uint16_t* dst = a.out + (((int64_t)s * a.tq + tau) * a.h_q + j * a.group + (c - tau * a.group)) * D;
#pragma unroll
    for (int e2 = 0; e2 < E / 2; ++e2)
      reinterpret_cast<uint32_t*>(dst + r * E)[e2] =
          DT::narrow(o[2 * e2] / l) | (DT::narrow(o[2 * e2 + 1] / l) << 16);
  }
}

// ------------------------------------------------------- balanced kernel --
//
// Persistent grid of W workgroups.  The (sequence, head group) ranges are
// laid end to end in 32-token tiles (range (s, g) holds ceil(L_s / 32)
// tiles, at least one); workgroup w owns the tiles [w C, (w+1) C) with
// C = max(ceil(total / W), kMinChunkTiles).  A range is processed by the
// workgroups whose shares it overlaps, one segment each; a range of at most
// v1_max_ctx tokens is never split and belongs to the workgroup its first tile
// falls in.  A range that ends up in one segment is written directly; the
// segments of a split range write fp32 partials to per-workgroup slots
// (2w for the range the share starts in, 2w + 1 for the one it ends in) and
// the range's first segment records (first workgroup, last workgroup, first
// slot) for the merge kernel; with a contiguous cache every range has the same
// length, and the merge kernel computes the record instead.

// The prefix lives in LDS, which the compiler treats as per-lane data; every
// lane reads the same entry, so readfirstlane keeps the scheduling arithmetic
// (and everything derived from it) in scalar registers.
template <bool PAGED>
__device__ __forceinline__ int64_t range_prefix(const Params& a, const int32_t* pref, int s) {
  if constexpr (PAGED)
    return __builtin_amdgcn_readfirstlane(pref[s]);
  else
    return (int64_t)s * a.n_groups * seq_tiles(a.s_kv);
}

// VC > 0 selects the vector-ALU segment code with VC columns (wave_segment_dot2).
template <class DT, int D, bool PAGED, bool XS, bool SPLIT, bool FUSED, int VC = 0>
__global__ __launch_bounds__(max_heads_per_group(D) * 64) void partition_balanced_kernel(Params a) {
  static_assert(VC == 0 || (D == kDot2D && !XS && !SPLIT && !FUSED), "vector-ALU variant shape");
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];   // wave tiles, then the prefix
  __shared__ int32_t wave_tot[kMaxHeadsPerGroup];
  __shared__ float2 mlx[kMaxHeadsPerGroup * 16];                     // sub-wave (m, l) exchange
  __shared__ int last_of_range;                                      // fused merge
  __shared__ int first_seq;                                          // paged: the share's first sequence
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;                // = hpw * wph
  // per-wave tiles: V staging (row layout) and the sub-wave state exchange;
  // the x-split layout with one wave per head needs neither
  // SPLIT (one or two KV heads, one head's 256 B of each token row per wave):
  // K goes through LDS as well (wave_segment's KD)
  constexpr bool KDB = SPLIT && !XS && D <= 128;
  constexpr int tile_elems =
      VC > 0 ? dot2_wave_elems(VC) : (XS && !SPLIT) ? 0 : wave_lds_elems<D, XS, KDB>();
  uint16_t* const vt = smem + w * tile_elems;
  int32_t* const pref = reinterpret_cast<int32_t*>(smem + nw * tile_elems);

  // ---- paged: pref[s] = n_groups * (tiles of sequences < s); arithmetic when
  // contiguous.  The host keeps every tile count of a balanced launch below
  // 2^30, so the share arithmetic below divides in 32 bits (a 64-bit division
  // is a long instruction sequence, and this prologue runs before a
  // workgroup's first K/V load).
  uint32_t total;
  if constexpr (PAGED) {
    int32_t run = 0;
    for (int base = 0; base < a.num_seqs; base += blockDim.x) {
      const int s = base + threadIdx.x;
      int32_t v = 0;
      if (s < a.num_seqs) {
        const int L = min(max(a.ctx_lens[s], 0), a.max_ctx);
        v = a.n_groups * seq_tiles(L);
      }
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int32_t t = __shfl_up(v, off);
        if (lane >= off) v += t;
      }
      if (lane == 63) wave_tot[w] = v;
      __syncthreads();
      int32_t before = run;
      for (int u = 0; u < w; ++u) before += wave_tot[u];
      if (s < a.num_seqs) pref[s + 1] = before + v;
      for (int u = 0; u < nw; ++u) run += wave_tot[u];
      __syncthreads();
    }
    if (threadIdx.x == 0) pref[0] = 0;
    __syncthreads();
    total = __builtin_amdgcn_readfirstlane(run);
  } else {
    total = (uint32_t)a.num_seqs * a.n_groups * seq_tiles(a.s_kv);
  }

  // share size (a contiguous cache's is the host's, which the merge uses too)
  const uint32_t chunk32 =
      PAGED ? max((total + gridDim.x - 1) / gridDim.x, (uint32_t)kMinChunkTiles) : (uint32_t)a.pchunk;
  const int64_t chunk = chunk32;
  const int64_t x0 = (int64_t)blockIdx.x * chunk;
  if (x0 >= total) return;                       // uniform: no share
  const int64_t x1 = min(x0 + chunk, (int64_t)total);

  // ---- first sequence whose ranges reach past x0 (the s with pref[s] <= x0 <
  // pref[s + 1]; pref rises by at least n_groups per sequence, so exactly one)
  int s, hg, L, nt;
  if constexpr (PAGED) {
    for (int t = threadIdx.x; t < a.num_seqs; t += blockDim.x)
      if (pref[t] <= x0 && x0 < pref[t + 1]) first_seq = t;
    __syncthreads();
    s = __builtin_amdgcn_readfirstlane(first_seq);
    L = seq_len<PAGED>(a, s);
    nt = seq_tiles(L);
    hg = (int)((uint32_t)(x0 - range_prefix<PAGED>(a, pref, s)) / (uint32_t)nt);
  } else {
    L = a.s_kv;
    nt = seq_tiles(L);
    const uint32_t per_seq = (uint32_t)a.n_groups * nt;   // tiles of one sequence
    s = (int)((uint32_t)x0 / per_seq);
    hg = (int)(((uint32_t)x0 - (uint32_t)s * per_seq) / (uint32_t)nt);
  }
  const int wg = blockIdx.x;
  const int heads = a.hpw * a.ncol;              // partial rows per slot: (KV head, column)
  const int wj = SPLIT ? w - (int)a.hpw_div.div(w) * a.hpw : w;   // the wave's head in the group

  for (;;) {
    const int64_t rs = range_prefix<PAGED>(a, pref, s) + (int64_t)hg * nt;
    if (rs >= x1) break;
    const int64_t re = rs + nt;
    const int r = s * a.n_groups + hg;
    const int j = hg * a.hpw + wj;
    // This workgroup's part of the range: nothing (an unsplit range it does not
    // own), the whole range (written directly), or one segment of a split range
    // (a partial).  One call site keeps a single copy of the segment code.
    bool run = true, complete = true;
    int t0 = 0, t1 = L, slot = 0;
    if (L <= a.v1_max_ctx) {
      run = rs >= x0;                            // never split: owned by its first tile's share
    } else {
      const int64_t sa = max(rs, x0) - rs;
      const int64_t sb = min(re, x1) - rs;
      t0 = (int)(sa * kTile);
      t1 = (int)min(sb * kTile, (int64_t)L);
      complete = sa == 0 && sb == nt;
      slot = 2 * wg + (rs <= x0 ? 0 : 1);
    }
    if (run) {
      const int64_t hrow = (int64_t)slot * heads + wj * a.ncol;
      float2* const pml = complete ? nullptr : a.part_ml + hrow;
      float* const po = complete ? nullptr : a.part_o + hrow * D;
      if constexpr (VC > 0)
        wave_segment_dot2<DT, PAGED, VC>(a, vt, s, j, t0, t1, complete, pml, 1, po, D);
      else
        wave_segment<DT, D, PAGED, XS, true, SPLIT, KDB, FUSED>(a, smem, vt, mlx, s, j, t0, t1,
                                                                complete, pml, 1, po, D);
      // (a contiguous cache's records are arithmetic: the merge recomputes them)
      if (PAGED && threadIdx.x == 0) {
        if (complete) {
          if (a.desc) a.desc[r] = make_int4(wg, wg, -1, 0);
        } else if (t0 == 0) {
          a.desc[r] = make_int4(wg, (int)((uint32_t)(re - 1) / chunk32), slot, 0);
        }
      }
      if (FUSED && !complete) {
        // Fused merge.  Publish this workgroup's partials, count it in, and
        // let the workgroup that completes the count merge the range; it
        // resets the counter for the next call.  Nothing waits on other
        // workgroups.  The partials were written with device-coherent stores
        // and are read with device-coherent loads, so no device-scope fence is
        // needed (on this part one writes back or invalidates the whole L2 of
        // the XCD): each wave waits until its stores have completed, the
        // barrier then orders them before thread 0's device-scope atomic, and
        // the merging waves issue their loads only after that atomic returned.
        const int wg0 = (int)((uint32_t)rs / chunk32);   // the range's first and last shares
        const int n = (int)((uint32_t)(re - 1) / chunk32) - wg0 + 1;
        wait_tile_loads();                       // vmcnt(0): loads and stores
        __syncthreads();
        if (threadIdx.x == 0)
          last_of_range = __hip_atomic_fetch_add(a.cnt + r, 1, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT) == n - 1;
        __syncthreads();
        if (last_of_range) {
          const int first = 2 * wg0 + (rs == (int64_t)wg0 * chunk ? 0 : 1);
          fused_range_merge<DT, D>(a, s, hg, wg0, n, first);
          if (threadIdx.x == 0)
            __hip_atomic_store(a.cnt + r, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();                         // last_of_range read before it is rewritten
      }
    }
    if (++hg == a.n_groups) {
      hg = 0;
      if (++s == a.num_seqs) break;
      L = seq_len<PAGED>(a, s);
      nt = seq_tiles(L);
    }
  }
}

// ----------------------------------------------------------- merge kernel --
//
// A head whose sequence was split is merged here: the n-ary form of the
// decode-long page's "_merge_running" over its n partials, then its "Final
// normalise + store".  The unit of work is a slot of 16 lanes; lane r of a
// slot holds d elements [r*D/16, (r+1)*D/16) of one partial row, so a slot
// reads a whole row per partial with 16-byte loads.  A head gets SPI slots
// (1, 4, 16 or 64, chosen by the host from the expected number of partials);
// slot u folds partials u, u + SPI, ... with a running maximum, eight loads
// in flight, and the SPI slot results are combined in slot order through
// LDS, so the result does not depend on scheduling.

constexpr int kMergeLanes = 16;                   // lanes per slot
constexpr int kMergeUnroll = 8;                   // partials in flight per slot
constexpr int kMergeSliceBelowBlocks = 256;       // slice d when the merge has fewer workgroups

// 256 threads, or one head of SPI slots when that is larger (SPI = 64: 1024)
__host__ __device__ constexpr int merge_block(int spi) {
  return spi * kMergeLanes > 256 ? spi * kMergeLanes : 256;
}
__host__ __device__ constexpr int merge_heads_per_block(int spi) {
  return merge_block(spi) / (kMergeLanes * spi);
}

// The record the balanced partition kernel would write for range r of a
// contiguous cache, computed instead of loaded (a load would be the merge's
// first dependent memory access): every range holds seq_tiles(s_kv) tiles and
// the host passes the share size.  Returns (first workgroup, last workgroup,
// first slot); a range written in one pass has first == last.  The balanced
// plan keeps the tile count below 2^30, and the divisions by the share size
// are a multiply and a shift with the host's constants (exact below 2^30).
__device__ __forceinline__ int4 contiguous_record(const Params& a, int r) {
  const uint32_t nt = (uint32_t)seq_tiles(a.s_kv);
  const uint32_t chunk = (uint32_t)a.pchunk;
  const uint32_t rs = (uint32_t)r * nt;
  const int wg0 = (int)a.pchunk_div.div(rs);
  const int wg1 = (int)a.pchunk_div.div(rs + nt - 1);
  if (a.s_kv <= a.v1_max_ctx || wg0 == wg1) return make_int4(wg0, wg0, -1, 0);
  return make_int4(wg0, wg1, 2 * wg0 + (rs == (uint32_t)wg0 * chunk ? 0 : 1), 0);
}

// SLICED: a head's d is cut into D / 32 slices of 32, each merged by its own
// slots (every slice reads all partials' (m, l), and its 128 bytes of each O
// row).  It multiplies the workgroups of a merge with few heads and many
// partials, whose reads would otherwise crowd onto few CUs.
template <class DT, int D, bool PAGED, bool BALANCED, int SPI, bool SLICED>
__global__ __launch_bounds__(merge_block(SPI)) void merge_kernel(Params a) {
  constexpr int NSL = SLICED ? D / 32 : 1;        // d slices per head
  constexpr int DS = D / NSL;                     // d per slice
  constexpr int E = DS / kMergeLanes;             // floats per lane: 2, 4, 8 or 16
  constexpr int VE = E < 4 ? E : 4;               // floats per load
  typedef float vecE_t __attribute__((ext_vector_type(VE)));
  // a 1024-thread block leaves 128 registers per lane: fewer loads in flight at d = 256
  constexpr int U = (merge_block(SPI) > 256 && E > 8) ? kMergeUnroll / 2 : kMergeUnroll;
  constexpr int SLOTS = merge_block(SPI) / kMergeLanes;
  constexpr int HPB = merge_heads_per_block(SPI);
  static_assert(E % 2 == 0 && HPB >= 1 && HPB * SPI == SLOTS, "merge shape");
  const int slot = threadIdx.x / kMergeLanes;
  const int r = threadIdx.x % kMergeLanes;
  const int sub = slot % SPI;                     // subset of the partials
  // one output row: (sequence s, query token tau, query head i) = item, the
  // row-major index of out[num_seqs, T_q, h_q]; slice: its d range
  const int vitem = blockIdx.x * HPB + slot / SPI;
  const int item = vitem / NSL;
  const int d0 = (vitem % NSL) * DS;
  const int heads = a.hpw * a.ncol;               // partial rows per balanced slot
  // ---- the partial rows of this head; n = 0 for a head written in one pass.
  // No early return: with SPI > 1 every slot reaches the barrier below.
  int n = 0, s = 0, local = 0;
  int64_t base = 0;
  int4 d{0, 0, 0, 0};
  const int rows_per_seq = a.tq * a.h_q;
  if (item < a.num_seqs * rows_per_seq) {        // (the host keeps this below 2^30)
    s = (int)a.rows_div.div(item);
    const int rem = item - s * rows_per_seq;      // tau * h_q + i
    const int tau = (int)a.hq_div.div(rem);
    const int i = rem - tau * a.h_q;
    const int j = (int)a.g_div.div(i);            // KV head
    const int c = tau * a.group + (i - j * a.group);   // column of KV head j's partial rows
    if constexpr (BALANCED) {
      const int hg = (int)a.hpw_div.div(j);       // head group
      if constexpr (PAGED)
        d = a.desc[s * a.n_groups + hg];
      else
        d = contiguous_record(a, s * a.n_groups + hg);
      n = d.y == d.x ? 0 : d.y - d.x + 1;
      local = (j - hg * a.hpw) * a.ncol + c;
    } else {
      const int L = seq_len<PAGED>(a, s);
      n = L <= a.v1_max_ctx ? 0 : (L + a.part_size - 1) / a.part_size;
      base = (((int64_t)s * a.h_kv + j) * a.ncol + c) * a.max_parts;
    }
  }
  auto row = [&](int k) -> int64_t {
    if constexpr (BALANCED)
      return (int64_t)(k == 0 ? d.z : 2 * (d.x + k)) * heads + local;
    else
      return base + k;
  };
  // ---- running (m, l, o) of this slot's subset, log2 units; empty = (-inf, 0, 0)
  float m = -INFINITY, l = 0.f;
  float o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;
  for (int k0 = sub; k0 < n; k0 += U * SPI) {
    float2 t2[U];
    vecE_t v[U][E / VE];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (k0 + u * SPI < n) {
        const int64_t rw = row(k0 + u * SPI);
        t2[u] = a.part_ml[rw];
        const vecE_t* src = reinterpret_cast<const vecE_t*>(a.part_o + rw * D + d0 + r * E);
#pragma unroll
        for (int e4 = 0; e4 < E / VE; ++e4) v[u][e4] = src[e4];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (k0 + u * SPI < n) {
        const float m_new = fmaxf(m, t2[u].x);    // finite: a partial holds at least one token
        const float a_old = __builtin_amdgcn_exp2f(m - m_new);
        const float a_new = __builtin_amdgcn_exp2f(t2[u].x - m_new);
        l = l * a_old + t2[u].y * a_new;
#pragma unroll
        for (int e4 = 0; e4 < E / VE; ++e4)
#pragma unroll
          for (int c = 0; c < VE; ++c)
            o[VE * e4 + c] = o[VE * e4 + c] * a_old + v[u][e4][c] * a_new;
        m = m_new;
      }
    }
  }
  uint16_t* dst = a.out + (int64_t)item * D + d0;
  if constexpr (SPI == 1) {
    if (n > 0) {
      uint32_t packed[E / 2];
#pragma unroll
      for (int e2 = 0; e2 < E / 2; ++e2)
        packed[e2] = DT::narrow(o[2 * e2] / l) | (DT::narrow(o[2 * e2 + 1] / l) << 16);
#pragma unroll
      for (int e2 = 0; e2 < E / 2; ++e2) reinterpret_cast<uint32_t*>(dst + r * E)[e2] = packed[e2];
    }
  } else {
    // ---- combine the SPI slot results of each head slice in slot order
    __shared__ float red_o[SLOTS][DS];
    __shared__ float red_m[SLOTS], red_l[SLOTS];
#pragma unroll
    for (int e = 0; e < E; ++e) red_o[slot][r * E + e] = o[e];
    if (r == 0) red_m[slot] = m;
    __syncthreads();
    const int first = slot - sub;                 // the head's first slot
    float sc = 0.f;                               // this slot's weight exp2(m_u - M)
    if (r == 0 && m != -INFINITY) {               // an empty subset (n < SPI) weighs 0
      float mm = -INFINITY;
      for (int u = 0; u < SPI; ++u) mm = fmaxf(mm, red_m[first + u]);
      sc = __builtin_amdgcn_exp2f(m - mm);
    }
    __syncthreads();
    if (r == 0) {
      red_m[slot] = sc;
      red_l[slot] = l * sc;
    }
    __syncthreads();
    if (n > 0) {
      float lsum = 0.f;
      for (int u = 0; u < SPI; ++u) lsum += red_l[first + u];
      for (int c = sub * kMergeLanes + r; c < DS; c += SPI * kMergeLanes) {
        float acc = 0.f;
        for (int u = 0; u < SPI; ++u) acc += red_o[first + u][c] * red_m[first + u];
        dst[c] = DT::narrow(acc / lsum);
      }
    }
  }
}

// ------------------------------------------------------------------ host --

// The device's scratch for gqa_decode_noalloc: partial triples and range
// records of the split sequences, GQA_NOALLOC_SCRATCH_BYTES per device, held
// by every device the library runs on until the process ends.  In host code
// `scratch` names a host-side stand-in, never the device memory: host code
// uses the address hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = GQA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device, looked up once per device.
gqa_status_t scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GQA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return GQA_ERR_LAUNCH;
    addr[dev] = p;
  }
  *out = addr[dev];
  return GQA_OK;
}

constexpr int32_t kDefaultV1Max = 256;
constexpr int32_t kFallbackPartition = 512;
// Fixed partitions: fewest work items (partition, head group, sequence) the
// host can count before it narrows the head groups: one per CU of an MI355X
// for a contiguous cache (equal items), four for a paged one (single-pass items
// of unknown lengths, which balance only when there are many).
constexpr int64_t kFixedMinItems = 256;
constexpr int64_t kFixedMinItemsPaged = 1024;
// Workgroups of a paged fixed-partition launch, at most: items beyond the grid
// are taken in further rounds.
constexpr int64_t kFixedGridCap = 2048;

struct Problem {
  bool paged;
  bool xsplit;        // paged caches in the x-split layout
  int tq;             // query tokens per sequence
  const void* q;
  const void* k;
  const void* v;
  void* out;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  int num_seqs;
  int max_blocks;
  int s_kv;
  int h_q;
  int h_kv;
  int d;
  int block_size;
  float scale;
  gqa_dtype_t dtype;
  void* ws;
  size_t ws_bytes;
  const gqa_policy_t* policy;
  void* stream;
  bool noalloc;       // workspace: the device's static scratch (gqa_decode_noalloc)
};

bool aligned(const void* ptr, uintptr_t n) { return (reinterpret_cast<uintptr_t>(ptr) & (n - 1)) == 0; }
size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

gqa_status_t resolve_policy(const gqa_policy_t* in, gqa_policy_t* out) {
  if (in == nullptr)
    gqa_policy_default(out);
  else
    *out = *in;
  const bool balanced = out->partition_size == 0;
  if ((!balanced && (out->partition_size < kTile || out->partition_size > (1 << 20) ||
                     out->partition_size % kTile != 0)) ||
      out->v1_max_ctx < 0 || out->phases < 0 || out->phases > 3 ||
      (out->flags & ~(GQA_POLICY_FUSED_MERGE | GQA_POLICY_VALU_DOT2)) != 0 ||
      ((out->flags & (GQA_POLICY_FUSED_MERGE | GQA_POLICY_VALU_DOT2)) && !balanced) ||
      ((out->flags & GQA_POLICY_FUSED_MERGE) && (out->flags & GQA_POLICY_VALU_DOT2)))
    return GQA_ERR_BAD_POLICY;
  if (out->phases == 0) out->phases = 3;
  return GQA_OK;
}

// KV heads per workgroup: the largest divisor of h_kv that is at most
// kGroupHeads (and max_heads_per_group(d)), so that a workgroup's waves read
// whole groups of adjacent heads of a token.  Four heads (1 KB of a 2 KB
// token row at d = 128, one workgroup of four waves per CU) beat eight on
// MI355X: a split range then spans half as many workgroups, so the launch
// writes half the fp32 partials, whose dirty lines the L2s must write back
// (contig_b8 step 29.6 -> 27.3 us, long_128k 92.9 -> 87.4 us, paged_b64
// 167.2 -> 163.5 us).  Two heads per workgroup were slower again.
constexpr int kGroupHeads = 4;
int heads_per_group(int h_kv, int d) {
  for (int h = std::min({h_kv, kGroupHeads, max_heads_per_group(d)}); h > 1; --h)
    if (h_kv % h == 0) return h;
  return 1;
}

// Waves of a balanced workgroup whose one or two KV heads split their
// segments.  Four waves, with K and V through LDS, beat eight waves with K in
// registers (same box, us per step: tiny_contig 5.8 -> 5.2; 64 paged sequences
// of 512-8192 tokens, 16/2 heads, 52.8-53.2 -> 50.7-51.4; 4 sequences of 32768
// tokens, 16/1 heads, 20.7 -> 19.6-20.0).
constexpr int kSplitWaves = 4;

// How a call is decomposed once the sizes are known.
struct Plan {
  bool balanced;
  int hpw;            // KV heads per workgroup
  int wph;            // waves per KV head: hpw * wph waves per workgroup
  int n_groups;       // h_kv / hpw
  int part_size;      // fixed mode
  int max_parts;      // fixed mode
  bool can_split;     // some sequence may exceed v1_max_ctx
  bool fused;         // split ranges merged by their last workgroup (no merge kernel)
  int vc;             // vector-ALU products with vc columns (4 or 8); 0: matrix cores
  bool paged;         // paged cache (the fixed decomposition then plans a work list)
  int hpw2;           // fixed, paged: KV heads per item of a split sequence
  size_t ws_desc, ws_cnt, ws_hdr, ws_items, ws_ml, ws_o, ws_total;   // workspace region bytes
};

int64_t upper_tiles(int num_seqs, int n_groups, int max_ctx) {
  return (int64_t)num_seqs * n_groups * std::max<int64_t>(1, ((int64_t)max_ctx + kTile - 1) / kTile);
}

// Byte sizes of the workspace regions.  The balanced decomposition gives each
// of its (at most grid_rows) workgroups two partial slots, plus a record per
// (sequence, head group); the fixed one has, for a paged cache, its work list
// (a header and up to one item per (sequence, KV head, partition)) and, when a
// sequence can be split, a partial slot per (sequence, query row, partition).
void size_workspace(Plan& pl, int num_seqs, int t_q, int h_q, int h_kv, int d, int64_t grid_rows) {
  pl.ws_desc = pl.ws_cnt = pl.ws_hdr = pl.ws_items = pl.ws_ml = pl.ws_o = 0;
  if (pl.balanced) {
    if (pl.can_split) {
      const size_t rows = (size_t)2 * grid_rows * pl.hpw * (h_q / h_kv) * t_q;
      pl.ws_desc = align256((size_t)num_seqs * pl.n_groups * sizeof(int4));
      pl.ws_cnt = pl.fused ? align256((size_t)num_seqs * pl.n_groups * sizeof(int)) : 0;
      pl.ws_ml = align256(rows * sizeof(float2));
      pl.ws_o = rows * (size_t)d * sizeof(float);
    }
  } else {
    if (pl.paged) {
      pl.ws_hdr = 256;
      pl.ws_items =
          align256((size_t)num_seqs * h_kv * (pl.can_split ? pl.max_parts : 1) * sizeof(int2));
    }
    if (pl.can_split) {
      const size_t rows = (size_t)num_seqs * h_q * t_q * pl.max_parts;
      pl.ws_ml = align256(rows * sizeof(float2));
      pl.ws_o = rows * (size_t)d * sizeof(float);
    }
  }
  pl.ws_total = pl.ws_desc + pl.ws_cnt + pl.ws_hdr + pl.ws_items + pl.ws_ml + pl.ws_o;
}

// Points the Params' workspace regions into ws (laid out as size_workspace says).
void place_workspace(Params& prm, const Plan& pl, char* ws) {
  size_t at = 0;
  auto take = [&](size_t n) -> char* { char* p = n ? ws + at : nullptr; at += n; return p; };
  prm.desc = reinterpret_cast<int4*>(take(pl.ws_desc));
  prm.cnt = reinterpret_cast<int*>(take(pl.ws_cnt));
  prm.fixed_hdr = reinterpret_cast<int*>(take(pl.ws_hdr));
  prm.items = reinterpret_cast<int2*>(take(pl.ws_items));
  prm.part_ml = reinterpret_cast<float2*>(take(pl.ws_ml));
  prm.part_o = reinterpret_cast<float*>(take(pl.ws_o));
}

// parts_per_seq: partitions every sequence is known to have (1 unless a
// contiguous cache is longer than v1_max_ctx); it only steers the head grouping
// of the fixed scheduler, never the workspace size.
Plan make_plan(int num_seqs, int t_q, int h_q, int h_kv, int d, int max_ctx,
               const gqa_policy_t& pol, bool paged, int64_t parts_per_seq = 1) {
  Plan pl{};
  pl.paged = paged;
  pl.hpw = heads_per_group(h_kv, d);
  // a workgroup of fewer than the full complement of waves gives each KV head
  // several waves, which split its segments (more loads in flight per head)
  pl.wph = 1;
  pl.n_groups = h_kv / pl.hpw;
  pl.can_split = max_ctx > pol.v1_max_ctx;
  // the balanced scheduler keeps its per-sequence prefix in LDS as int32
  pl.balanced = pol.partition_size == 0 && num_seqs <= kMaxSeqsBalanced &&
                upper_tiles(num_seqs, pl.n_groups, max_ctx) < (int64_t)INT32_MAX / 2;
  // Groups of one or two KV heads (small h_kv) get kSplitWaves / hpw waves per
  // head, which split each segment's tiles: a lone wave per head walking a
  // short sequence is latency-bound.  Larger groups have waves enough; on a
  // batch of 256 sequences of ~3400 tokens with four KV heads the split cost
  // 2%.
  if (pl.balanced && pl.hpw <= 2 && !(pol.flags & (GQA_POLICY_FUSED_MERGE | GQA_POLICY_VALU_DOT2)))
    pl.wph = kSplitWaves / pl.hpw;
  if (pl.balanced && (pol.flags & GQA_POLICY_VALU_DOT2))
    pl.vc = (h_q / h_kv) * t_q <= 4 ? 4 : 8;
  pl.part_size = pol.partition_size > 0 ? pol.partition_size : kFallbackPartition;
  pl.max_parts = pl.can_split ? (int)(((int64_t)max_ctx + pl.part_size - 1) / pl.part_size) : 1;
  if (!pl.balanced && !paged) {
    // One workgroup per (partition, head group, sequence).  With fewer work
    // items than kFixedMinItems (e.g. 8 unsplit sequences in two groups of four
    // KV heads: 16), narrow the head groups, down to one KV head per workgroup
    // as the pages have it; a group of one or two heads gives each head several
    // waves, which split its partition's tiles.
    while (pl.hpw > 1 && (int64_t)num_seqs * parts_per_seq * (h_kv / pl.hpw) < kFixedMinItems) {
      int h = pl.hpw - 1;
      while (h > 1 && h_kv % h != 0) --h;
      pl.hpw = h;
    }
    pl.n_groups = h_kv / pl.hpw;
    // as in the balanced scheduler, only groups of one or two heads split
    if (pl.hpw <= 2) pl.wph = max_heads_per_group(d) / pl.hpw;
  } else if (!pl.balanced) {
    // Paged: items of 1, 2 or 4 heads, so that the workgroup's waves divide
    // evenly among an item's heads.  Single-pass items narrow until the host
    // can count kFixedMinItemsPaged of them (every sequence may be a single
    // long pass, up to v1_max_ctx tokens); partitions of split sequences are
    // short and take the widest group.
    const int waves = kFixedPagedWaves;
    auto pow2_group = [&](int cap) {
      int h = 1;
      while (2 * h <= std::min(cap, waves) && h_kv % (2 * h) == 0) h *= 2;
      return h;
    };
    pl.hpw2 = pow2_group(kGroupHeads);
    pl.hpw = pl.hpw2;
    while (pl.hpw > 1 && (int64_t)num_seqs * (h_kv / pl.hpw) < kFixedMinItemsPaged) pl.hpw /= 2;
    pl.n_groups = h_kv / pl.hpw;
    pl.wph = waves / pl.hpw;
  }
  pl.fused = pl.balanced && pl.can_split && (pol.flags & GQA_POLICY_FUSED_MERGE) != 0;
  size_workspace(pl, num_seqs, t_q, h_q, h_kv, d, kMaxGrid);
  return pl;
}

// Resident workgroups for a kernel, cached per (device, kernel, block, dynamic
// LDS rounded up to 4 KB); *cus_out receives the device's CU count.  The
// occupancy is queried for the rounded size, which never overstates it, so
// calls whose LDS differs by a few sequences of prefix share one entry.
int resident_grid(const void* kernel, int block, size_t dyn_lds_exact, int* cus_out = nullptr) {
  const size_t dyn_lds = (dyn_lds_exact + 4095) & ~(size_t)4095;
  struct Entry { int dev; const void* k; int block; size_t lds; int grid; int cus; };
  static std::mutex mu;
  static Entry cache[64];
  static int n_cache = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    for (int e = 0; e < n_cache; ++e)
      if (cache[e].dev == dev && cache[e].k == kernel && cache[e].block == block &&
          cache[e].lds == dyn_lds) {
        if (cus_out) *cus_out = cache[e].cus;
        return cache[e].grid;
      }
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, dyn_lds) != hipSuccess)
    return 0;
  const int grid = std::max(1, cus * std::max(1, per_cu));
  if (cus_out) *cus_out = cus;
  std::lock_guard<std::mutex> lock(mu);
  if (n_cache < 64) cache[n_cache++] = Entry{dev, kernel, block, dyn_lds, grid, cus};
  return grid;
}

// Per-wave LDS tiles: V staging (row layout) and the sub-wave state exchange.
template <int D, bool XS>
size_t tiles_lds(const Plan& pl) {
  if (pl.vc > 0) return (size_t)pl.hpw * dot2_wave_elems(pl.vc) * sizeof(uint16_t);
  if (pl.balanced && pl.wph > 1 && !XS && D <= 128)   // split: K through LDS too
    return (size_t)pl.hpw * pl.wph * wave_lds_elems<D, XS, true>() * sizeof(uint16_t);
  return (XS && pl.wph == 1) ? 0
                             : (size_t)pl.hpw * pl.wph * wave_lds_elems<D, XS>() * sizeof(uint16_t);
}

template <class DT, int D, bool PAGED, bool XS>
const void* balanced_kernel(const Plan& pl) {
  if constexpr (D == kDot2D && !XS) {
    if (pl.vc == 4)
      return reinterpret_cast<const void*>(&partition_balanced_kernel<DT, D, PAGED, XS, false, false, 4>);
    if (pl.vc == 8)
      return reinterpret_cast<const void*>(&partition_balanced_kernel<DT, D, PAGED, XS, false, false, 8>);
  }
  if (pl.fused)   // one wave per head (make_plan)
    return reinterpret_cast<const void*>(&partition_balanced_kernel<DT, D, PAGED, XS, false, true>);
  return pl.wph > 1
             ? reinterpret_cast<const void*>(&partition_balanced_kernel<DT, D, PAGED, XS, true, false>)
             : reinterpret_cast<const void*>(&partition_balanced_kernel<DT, D, PAGED, XS, false, false>);
}

template <int D, bool PAGED, bool XS>
size_t balanced_lds(const Params& prm, const Plan& pl) {
  return tiles_lds<D, XS>(pl) +
         (PAGED ? (size_t)(prm.num_seqs + 1) * sizeof(int32_t) : 0);
}

// Workgroups of a persistent launch of `waves`-wave workgroups: enough for
// kWavesPerCu waves on every CU (one workgroup per CU when it has that many
// waves), at most as many as fit at once.  0 if the device cannot be queried.
int persistent_grid(const void* kern, int waves, size_t dyn_lds) {
  int cus = 0;
  const int resident = resident_grid(kern, 64 * waves, dyn_lds, &cus);
  if (resident <= 0) return 0;
  const int per_cu = std::max(1, (kWavesPerCu + waves - 1) / waves);
  return std::min(resident, std::max(1, cus) * per_cu);
}

// Workgroups of the balanced partition launch: enough for kWavesPerCu waves
// on every CU (one workgroup per CU when it has that many waves), at most the
// resident count and kMaxGrid, and no more than gives every workgroup
// kMinChunkTiles tiles.  More workgroups than that read no faster (4 waves of
// two 16 KB tiles in flight already saturate a CU's share of HBM) but split
// sequences into more partials for the merge.
template <class DT, int D, bool PAGED, bool XS>
int balanced_grid(const Params& prm, const Plan& pl) {
  const int resident = persistent_grid(balanced_kernel<DT, D, PAGED, XS>(pl), pl.hpw * pl.wph,
                                       balanced_lds<D, PAGED, XS>(prm, pl));
  if (resident <= 0) return 0;
  const int64_t want =
      (upper_tiles(prm.num_seqs, pl.n_groups, prm.max_ctx) + kMinChunkTiles - 1) / kMinChunkTiles;
  return (int)std::max<int64_t>(1, std::min<int64_t>({(int64_t)kMaxGrid, resident, want}));
}

template <class DT, int D, bool PAGED, int SPI, bool SLICED>
gqa_status_t launch_merge(bool balanced, int64_t items, void** args, hipStream_t stream) {
  const void* kern =
      balanced ? reinterpret_cast<const void*>(&merge_kernel<DT, D, PAGED, true, SPI, SLICED>)
               : reinterpret_cast<const void*>(&merge_kernel<DT, D, PAGED, false, SPI, SLICED>);
  constexpr int per_block = merge_heads_per_block(SPI);
  const int64_t vitems = items * (SLICED ? D / 32 : 1);
  const int64_t grid = (vitems + per_block - 1) / per_block;
  if (hipLaunchKernel(kern, dim3((unsigned)grid), dim3(merge_block(SPI)), args, 0, stream) !=
      hipSuccess)
    return GQA_ERR_LAUNCH;
  return GQA_OK;
}

// scratch: non-null for gqa_decode_noalloc, the device address of the static
// scratch array; the workspace is then sized for the actual grid and placed there.
template <class DT, int D, bool PAGED, bool XS>
gqa_status_t launch_typed(const Params& prm, const Plan& pl, int phases, hipStream_t stream,
                          char* scratch) {
  Params local = prm;
  void* args[] = {&local};
  const int block = 64 * pl.hpw * pl.wph;
  int grid_b = 0;                                 // balanced partition grid
  if (pl.balanced) {
    grid_b = balanced_grid<DT, D, PAGED, XS>(prm, pl);
    if (grid_b <= 0) return GQA_ERR_LAUNCH;
  }
  if (scratch && pl.ws_total > 0) {
    Plan sized = pl;
    if (pl.balanced)
      size_workspace(sized, prm.num_seqs, prm.tq, prm.h_q, prm.h_kv, D, grid_b);
    if (sized.ws_total > kScratchBytes) return GQA_ERR_WORKSPACE;
    place_workspace(local, sized, scratch);
  }
  if (pl.balanced) {
    if (!PAGED) {
      // the share size the partition kernel derives, for the merge kernel
      const int64_t total = (int64_t)prm.num_seqs * pl.n_groups *
                            std::max<int64_t>(1, ((int64_t)prm.s_kv + kTile - 1) / kTile);
      const int64_t chunk = std::max<int64_t>((total + grid_b - 1) / grid_b, kMinChunkTiles);
      local.pchunk = (int)chunk;
      local.pchunk_div = fast_div((uint32_t)chunk);
    }
  }
  if (phases & 1) {
    if (pl.balanced) {
      const void* kern = balanced_kernel<DT, D, PAGED, XS>(pl);
      if (hipLaunchKernel(kern, dim3(grid_b), dim3(block), args,
                          balanced_lds<D, PAGED, XS>(prm, pl), stream) != hipSuccess)
        return GQA_ERR_LAUNCH;
    } else if constexpr (PAGED) {
      // the work list, then items blockIdx.x, blockIdx.x + grid, ... of it
      if (hipLaunchKernel(reinterpret_cast<const void*>(&fixed_plan_kernel), dim3(1),
                          dim3(kPlanThreads), args, 0, stream) != hipSuccess)
        return GQA_ERR_LAUNCH;
      const int64_t bound = (int64_t)prm.num_seqs * prm.h_kv * pl.max_parts;   // items, at most
      const int grid = (int)std::min(bound, kFixedGridCap);
      if (hipLaunchKernel(reinterpret_cast<const void*>(&partition_fixed_paged_kernel<DT, D, XS>),
                          dim3(grid), dim3(64 * kFixedPagedWaves), args,
                          std::max(kFixedPagedLds,
                                   (size_t)kFixedPagedWaves *
                                       wave_lds_elems<D, XS, fixed_paged_kd(D, XS)>() *
                                       sizeof(uint16_t)),
                          stream) != hipSuccess)
        return GQA_ERR_LAUNCH;
    } else {
      const int64_t grid = (int64_t)pl.max_parts * pl.n_groups * prm.num_seqs;
      // Non-temporal loads unless some wave may walk more than one partition's
      // worth of tokens in a single pass (a sequence of up to v1_max_ctx tokens
      // that is not split).
      const bool short_walks = prm.v1_max_ctx <= prm.part_size || prm.s_kv > prm.v1_max_ctx;
      const bool sw = pl.wph > 1;
      const void* kern =
          short_walks
              ? (sw ? reinterpret_cast<const void*>(&partition_fixed_kernel<DT, D, XS, true, true>)
                    : reinterpret_cast<const void*>(&partition_fixed_kernel<DT, D, XS, true, false>))
              : (sw ? reinterpret_cast<const void*>(&partition_fixed_kernel<DT, D, XS, false, true>)
                    : reinterpret_cast<const void*>(&partition_fixed_kernel<DT, D, XS, false, false>));
      if (hipLaunchKernel(kern, dim3((unsigned)grid), dim3(block), args, tiles_lds<D, XS>(pl),
                          stream) != hipSuccess)
        return GQA_ERR_LAUNCH;
    }
  }
  if ((phases & 2) && pl.can_split && !pl.fused) {
    // partials per split head: about grid / ranges for the balanced scheduler
    // (a range's tiles spread over that many shares), max_parts for fixed partitions
    int64_t per_head = pl.max_parts;
    if (pl.balanced) {
      const int64_t ranges = std::max<int64_t>(1, (int64_t)prm.num_seqs * pl.n_groups);
      per_head = (grid_b + ranges - 1) / ranges + 1;
    }
    const int64_t items = (int64_t)prm.num_seqs * prm.tq * prm.h_q;
    // Slots per head: enough that a slot folds at most two batches of partials
    // and that the launch has 4096 slots or more (1024 waves), at most 16
    // unless a head has more than 512 partials.
    int spi = 1;
    while (spi < 16 && (per_head > 2 * kMergeUnroll * spi || items * spi < 4096)) spi *= 4;
    if (per_head > 16 * 4 * kMergeUnroll) spi = 64;
    // Few heads with many partials would leave most CUs idle: cut each head's
    // d into slices of 32 when the unsliced grid has fewer workgroups than CUs.
    const int64_t blocks = (items + merge_heads_per_block(spi) - 1) / merge_heads_per_block(spi);
    const bool sliced = spi >= 16 && blocks < kMergeSliceBelowBlocks;
    gqa_status_t st;
    switch (spi) {
      case 1: st = launch_merge<DT, D, PAGED, 1, false>(pl.balanced, items, args, stream); break;
      case 4: st = launch_merge<DT, D, PAGED, 4, false>(pl.balanced, items, args, stream); break;
      case 16:
        st = sliced ? launch_merge<DT, D, PAGED, 16, true>(pl.balanced, items, args, stream)
                    : launch_merge<DT, D, PAGED, 16, false>(pl.balanced, items, args, stream);
        break;
      default:
        st = sliced ? launch_merge<DT, D, PAGED, 64, true>(pl.balanced, items, args, stream)
                    : launch_merge<DT, D, PAGED, 64, false>(pl.balanced, items, args, stream);
        break;
    }
    if (st != GQA_OK) return st;
  }
  return GQA_OK;
}

template <class DT, int D>
gqa_status_t launch_layout(const Problem& pb, const Params& prm, const Plan& pl, int ph,
                           hipStream_t st, char* scr) {
  if (pb.xsplit) return launch_typed<DT, D, true, true>(prm, pl, ph, st, scr);
  return pb.paged ? launch_typed<DT, D, true, false>(prm, pl, ph, st, scr)
                  : launch_typed<DT, D, false, false>(prm, pl, ph, st, scr);
}

template <class DT>
gqa_status_t launch_dtype(const Problem& pb, const Params& prm, const Plan& pl, int ph,
                          hipStream_t st, char* scr) {
  if (pb.d == 64) return launch_layout<DT, 64>(pb, prm, pl, ph, st, scr);
  if (pb.d == 128) return launch_layout<DT, 128>(pb, prm, pl, ph, st, scr);
  return launch_layout<DT, 256>(pb, prm, pl, ph, st, scr);
}

gqa_status_t run(const Problem& pb) {
  // ---- sizes, shapes, support (no HIP call before every check has passed)
  if (pb.num_seqs < 0 || pb.h_q <= 0 || pb.h_kv <= 0 || pb.h_q % pb.h_kv != 0)
    return GQA_ERR_BAD_SHAPE;
  if (pb.paged ? (pb.max_blocks <= 0) : (pb.s_kv < 0)) return GQA_ERR_BAD_SHAPE;
  if (pb.dtype != GQA_F16 && pb.dtype != GQA_BF16) return GQA_ERR_UNSUPPORTED;
  if (pb.d != 64 && pb.d != 128 && pb.d != 256) return GQA_ERR_UNSUPPORTED;
  const int G = pb.h_q / pb.h_kv;
  if (pb.tq < 1) return GQA_ERR_BAD_SHAPE;
  if (G * pb.tq > 16) return GQA_ERR_UNSUPPORTED;
  int bs_shift = 0;
  if (pb.paged) {
    if (pb.block_size < 16 || pb.block_size > 256 || (pb.block_size & (pb.block_size - 1)))
      return GQA_ERR_UNSUPPORTED;
    while ((1 << bs_shift) < pb.block_size) ++bs_shift;
  }
  if (!isfinite(pb.scale)) return GQA_ERR_BAD_SCALE;
  gqa_policy_t pol;
  const gqa_status_t ps = resolve_policy(pb.policy, &pol);
  if (ps != GQA_OK) return ps;
  const int64_t max_ctx64 = pb.paged ? (int64_t)pb.max_blocks * pb.block_size : pb.s_kv;
  if (max_ctx64 > (1 << 30)) return GQA_ERR_BAD_SHAPE;
  const int max_ctx = (int)max_ctx64;
  if ((pol.flags & GQA_POLICY_VALU_DOT2) && (pb.d != kDot2D || pb.xsplit || G * pb.tq > 8))
    return GQA_ERR_UNSUPPORTED;
  const int64_t parts_per_seq =
      (!pb.paged && pol.partition_size > 0 && pb.s_kv > pol.v1_max_ctx)
          ? ((int64_t)pb.s_kv + pol.partition_size - 1) / pol.partition_size
          : 1;
  const Plan pl =
      make_plan(pb.num_seqs, pb.tq, pb.h_q, pb.h_kv, pb.d, max_ctx, pol, pb.paged, parts_per_seq);
  if ((pol.flags & GQA_POLICY_VALU_DOT2) && !pl.balanced) return GQA_ERR_UNSUPPORTED;
  if (!pl.balanced && (int64_t)pl.max_parts * pb.h_kv * pb.num_seqs > INT32_MAX)
    return GQA_ERR_BAD_SHAPE;
  // query rows below 2^30: the kernels split row indices with FastDiv
  if ((int64_t)pb.h_q * pb.tq * pb.num_seqs >= (int64_t(1) << 30)) return GQA_ERR_BAD_SHAPE;
  if (pb.num_seqs == 0) return GQA_OK;

  // ---- pointers
  // an empty contiguous cache (s_kv == 0) is never read, so its pointers may be NULL
  const bool reads_kv = pb.paged || pb.s_kv > 0;
  if (!pb.q || !pb.out || (reads_kv && (!pb.k || !pb.v))) return GQA_ERR_NULL_PTR;
  if (pb.paged && (!pb.block_table || !pb.ctx_lens)) return GQA_ERR_NULL_PTR;
  if (!aligned(pb.q, 16) || !aligned(pb.k, 16) || !aligned(pb.v, 16) || !aligned(pb.out, 16))
    return GQA_ERR_MISALIGNED;
  if (pb.paged && (!aligned(pb.block_table, 4) || !aligned(pb.ctx_lens, 4)))
    return GQA_ERR_MISALIGNED;
  if (pb.noalloc) {
    // the workspace is the device's static scratch; the fused merge's counters
    // would need it zeroed first, so that flag is not offered here
    if (pol.flags & GQA_POLICY_FUSED_MERGE) return GQA_ERR_UNSUPPORTED;
    if (!pl.balanced && pl.ws_total > kScratchBytes) return GQA_ERR_WORKSPACE;
  } else if (pl.ws_total > 0) {
    if (!pb.ws || pb.ws_bytes < pl.ws_total) return GQA_ERR_WORKSPACE;
    if (!aligned(pb.ws, 256)) return GQA_ERR_MISALIGNED;
  }

  // ---- launch
  Params prm{};
  prm.q = static_cast<const uint16_t*>(pb.q);
  prm.k = static_cast<const uint16_t*>(pb.k);
  prm.v = static_cast<const uint16_t*>(pb.v);
  prm.out = static_cast<uint16_t*>(pb.out);
  prm.block_table = pb.block_table;
  prm.ctx_lens = pb.ctx_lens;
  if (pl.ws_total > 0 && !pb.noalloc) place_workspace(prm, pl, static_cast<char*>(pb.ws));
  prm.num_seqs = pb.num_seqs;
  prm.h_q = pb.h_q;
  prm.h_kv = pb.h_kv;
  prm.group = G;
  prm.tq = pb.tq;
  prm.ncol = G * pb.tq;
  prm.hpw = pl.hpw;
  prm.wph = pl.wph;
  prm.n_groups = pl.n_groups;
  prm.s_kv = pb.s_kv;
  prm.max_blocks = pb.max_blocks;
  prm.bs_shift = bs_shift;
  prm.max_ctx = max_ctx;
  prm.part_size = pl.part_size;
  // with no workspace nothing may split: the single-pass bound covers every sequence
  prm.v1_max_ctx = pl.can_split ? pol.v1_max_ctx : max_ctx;
  prm.max_parts = pl.max_parts;
  // fixed mode, paged: size classes of the planner's sort, (item tiles x heads) >> plan_shift
  prm.hpw2 = pl.hpw2;
  if (!pl.balanced && pb.paged) {
    const int64_t v1_tiles = ((int64_t)std::min(prm.v1_max_ctx, max_ctx) + kTile - 1) / kTile;
    const int64_t part_tiles = ((int64_t)pl.part_size + kTile - 1) / kTile;
    int64_t largest = std::max(v1_tiles * pl.hpw, part_tiles * pl.hpw2);
    while (largest >= kPlanBuckets) {
      largest >>= 1;
      ++prm.plan_shift;
    }
  }
  prm.c = pb.scale * kLog2e;
  prm.rows_div = fast_div((uint32_t)(pb.tq * pb.h_q));
  prm.hq_div = fast_div((uint32_t)pb.h_q);
  prm.g_div = fast_div((uint32_t)G);
  prm.hpw_div = fast_div((uint32_t)pl.hpw);
  hipStream_t st = static_cast<hipStream_t>(pb.stream);
  char* scr = nullptr;
  if (pb.noalloc) {
    void* addr = nullptr;
    const gqa_status_t ss = scratch_address(&addr);
    if (ss != GQA_OK) return ss;
    scr = static_cast<char*>(addr);
  }
  if (pb.dtype == GQA_F16) return launch_dtype<F16>(pb, prm, pl, pol.phases, st, scr);
  return launch_dtype<BF16>(pb, prm, pl, pol.phases, st, scr);
}

gqa_status_t run_paged(bool xsplit, bool noalloc, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_table, const int32_t* ctx_lens, void* out,
                       int num_seqs, int max_blocks_per_seq, int h_q, int h_kv, int d_head,
                       int block_size, float scale, gqa_dtype_t dtype, void* workspace,
                       size_t workspace_bytes, const gqa_policy_t* policy, void* stream) {
  Problem pb{};
  pb.paged = true;
  pb.xsplit = xsplit;
  pb.noalloc = noalloc;
  pb.tq = 1;
  pb.q = q;
  pb.k = k_cache;
  pb.v = v_cache;
  pb.out = out;
  pb.block_table = block_table;
  pb.ctx_lens = ctx_lens;
  pb.num_seqs = num_seqs;
  pb.max_blocks = max_blocks_per_seq;
  pb.h_q = h_q;
  pb.h_kv = h_kv;
  pb.d = d_head;
  pb.block_size = block_size;
  pb.scale = scale;
  pb.dtype = dtype;
  pb.ws = workspace;
  pb.ws_bytes = workspace_bytes;
  pb.policy = policy;
  pb.stream = stream;
  return run(pb);
}

}  // namespace

extern "C" {

void gqa_policy_default(gqa_policy_t* p) {
  if (!p) return;
  p->partition_size = 0;
  p->v1_max_ctx = kDefaultV1Max;
  p->phases = 0;
  p->flags = 0;
}

void gqa_policy_pages(gqa_policy_t* p) {
  if (!p) return;
  p->partition_size = 512;
  p->v1_max_ctx = 8192;
  p->phases = 0;
  p->flags = 0;
}

size_t gqa_decode_workspace_size(int num_seqs, int h_q, int h_kv, int d_head, int max_ctx,
                                 const gqa_policy_t* policy) {
  gqa_policy_t pol;
  if (resolve_policy(policy, &pol) != GQA_OK) return 0;
  if (num_seqs < 0 || h_q <= 0 || h_kv <= 0 || h_q % h_kv != 0 || d_head <= 0 || max_ctx < 0)
    return 0;
  return make_plan(num_seqs, 1, h_q, h_kv, d_head, max_ctx, pol, true).ws_total;
}

gqa_status_t gqa_decode(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_table, const int32_t* ctx_lens, void* out,
                        int num_seqs, int max_blocks_per_seq, int h_q, int h_kv,
                        int d_head, int block_size, float scale, gqa_dtype_t dtype,
                        void* workspace, size_t workspace_bytes,
                        const gqa_policy_t* policy, void* stream) {
  return run_paged(false, false, q, k_cache, v_cache, block_table, ctx_lens, out, num_seqs,
                   max_blocks_per_seq, h_q, h_kv, d_head, block_size, scale, dtype, workspace,
                   workspace_bytes, policy, stream);
}

gqa_status_t gqa_decode_xsplit(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* ctx_lens, void* out,
                               int num_seqs, int max_blocks_per_seq, int h_q, int h_kv,
                               int d_head, int block_size, float scale, gqa_dtype_t dtype,
                               void* workspace, size_t workspace_bytes,
                               const gqa_policy_t* policy, void* stream) {
  return run_paged(true, false, q, k_cache, v_cache, block_table, ctx_lens, out, num_seqs,
                   max_blocks_per_seq, h_q, h_kv, d_head, block_size, scale, dtype, workspace,
                   workspace_bytes, policy, stream);
}

gqa_status_t gqa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_table, const int32_t* ctx_lens, void* out,
                                int num_seqs, int max_blocks_per_seq, int h_q, int h_kv,
                                int d_head, int block_size, float scale, gqa_dtype_t dtype,
                                const gqa_policy_t* policy, void* stream) {
  return run_paged(false, true, q, k_cache, v_cache, block_table, ctx_lens, out, num_seqs,
                   max_blocks_per_seq, h_q, h_kv, d_head, block_size, scale, dtype, nullptr, 0,
                   policy, stream);
}

gqa_status_t gqa_decode_contiguous(const void* q, const void* k, const void* v, void* out,
                                   int num_seqs, int s_kv, int h_q, int h_kv, int d_head,
                                   float scale, gqa_dtype_t dtype,
                                   void* workspace, size_t workspace_bytes,
                                   const gqa_policy_t* policy, void* stream) {
  Problem pb{};
  pb.paged = false;
  pb.tq = 1;
  pb.q = q;
  pb.k = k;
  pb.v = v;
  pb.out = out;
  pb.num_seqs = num_seqs;
  pb.s_kv = s_kv;
  pb.h_q = h_q;
  pb.h_kv = h_kv;
  pb.d = d_head;
  pb.block_size = 16;
  pb.scale = scale;
  pb.dtype = dtype;
  pb.ws = workspace;
  pb.ws_bytes = workspace_bytes;
  pb.policy = policy;
  pb.stream = stream;
  return run(pb);
}

gqa_status_t gqa_decode_ex(const gqa_decode_args_t* args) {
  if (!args) return GQA_ERR_NULL_PTR;
  const gqa_decode_args_t& x = *args;
  if (x.layout != GQA_KV_CONTIGUOUS && x.layout != GQA_KV_PAGED && x.layout != GQA_KV_PAGED_XSPLIT)
    return GQA_ERR_UNSUPPORTED;
  Problem pb{};
  pb.paged = x.layout != GQA_KV_CONTIGUOUS;
  pb.xsplit = x.layout == GQA_KV_PAGED_XSPLIT;
  pb.tq = x.t_q;
  pb.q = x.q;
  pb.k = x.k;
  pb.v = x.v;
  pb.out = x.out;
  pb.block_table = x.block_table;
  pb.ctx_lens = x.ctx_lens;
  pb.num_seqs = x.num_seqs;
  pb.max_blocks = x.max_blocks_per_seq;
  pb.s_kv = x.s_kv;
  pb.h_q = x.h_q;
  pb.h_kv = x.h_kv;
  pb.d = x.d_head;
  pb.block_size = pb.paged ? x.block_size : 16;
  pb.scale = x.scale;
  pb.dtype = x.dtype;
  pb.ws = x.workspace;
  pb.ws_bytes = x.workspace_bytes;
  pb.policy = x.policy;
  pb.stream = x.stream;
  return run(pb);
}

size_t gqa_decode_ex_workspace_size(const gqa_decode_args_t* args) {
  if (!args) return 0;
  const gqa_decode_args_t& x = *args;
  gqa_policy_t pol;
  if (resolve_policy(x.policy, &pol) != GQA_OK) return 0;
  if (x.num_seqs < 0 || x.t_q < 1 || x.h_q <= 0 || x.h_kv <= 0 || x.h_q % x.h_kv != 0 ||
      x.d_head <= 0)
    return 0;
  int64_t max_ctx;
  if (x.layout == GQA_KV_CONTIGUOUS)
    max_ctx = x.s_kv;
  else if (x.layout == GQA_KV_PAGED || x.layout == GQA_KV_PAGED_XSPLIT)
    max_ctx = (int64_t)x.max_blocks_per_seq * x.block_size;
  else
    return 0;
  if (max_ctx < 0 || max_ctx > (1 << 30)) return 0;
  return make_plan(x.num_seqs, x.t_q, x.h_q, x.h_kv, x.d_head, (int)max_ctx, pol,
                   x.layout != GQA_KV_CONTIGUOUS).ws_total;
}

const char* gqa_status_string(gqa_status_t status) {
  switch (status) {
    case GQA_OK: return "GQA_OK: success";
    case GQA_ERR_NULL_PTR: return "GQA_ERR_NULL_PTR: a required pointer is NULL";
    case GQA_ERR_BAD_SHAPE: return "GQA_ERR_BAD_SHAPE: invalid or inconsistent sizes";
    case GQA_ERR_UNSUPPORTED: return "GQA_ERR_UNSUPPORTED: d_head, group size, block size or dtype not supported";
    case GQA_ERR_MISALIGNED: return "GQA_ERR_MISALIGNED: pointer alignment requirement not met";
    case GQA_ERR_WORKSPACE: return "GQA_ERR_WORKSPACE: workspace missing or too small (gqa_decode_noalloc: more than its static scratch)";
    case GQA_ERR_BAD_POLICY: return "GQA_ERR_BAD_POLICY: policy fields out of range";
    case GQA_ERR_BAD_SCALE: return "GQA_ERR_BAD_SCALE: scale is not finite";
    case GQA_ERR_LAUNCH: return "GQA_ERR_LAUNCH: kernel launch failed";
  }
  return "unknown gqa_status_t";
}

}  // extern "C"
