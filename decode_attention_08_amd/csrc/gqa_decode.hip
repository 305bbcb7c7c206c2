// Single-query GQA decode attention for MI355X (gfx950, CDNA4).
//
// Two kernels:
//   partition_kernel  one workgroup per (partition, KV head, sequence).  Its
//                     NW waves stream 32-token tiles of K and V from HBM and
//                     keep a running (m, l, O) for all G query heads sharing
//                     the KV head (decode-long page, "Local attention" tile
//                     sweep and "_merge_running").  At the end the waves are
//                     merged in LDS; a single-partition sequence is
//                     normalised and stored (kernel-map page,
//                     "paged_attention_v1"), a split one writes its fp32
//                     partial triple (kernel-map page, "paged_attention_v2").
//   merge_kernel      one wave per (sequence, query head) of a split sequence:
//                     the n-ary form of "_merge_running" followed by the
//                     decode-long page's "Final normalise + store".
//
// Matrix-core mapping (v_mfma_f32_16x16x32_{f16,bf16}, wave64).  The G <= 16
// query heads of one KV head are the 16-wide N side of both products, padded
// with zero query rows:
//   S^T[16 tok x 16 head] += K[16 tok x 32 d] . Q^T[32 d x 16 head]
//   O^T[16 d x 16 head]   += V^T[16 d x 32 tok] . P^T[32 tok x 16 head]
// With this orientation every lane owns one head column (lane % 16) in both
// the score and the output accumulators, so the online-softmax state of a
// head never leaves its lane group; only the tile max is exchanged between
// the four 16-lane groups.  K feeds the A operand straight from HBM with
// 16-byte loads (8 consecutive d of one token per lane).  V needs tokens
// along the operand's K side, so each wave stages its V tile in LDS with
// coalesced 16-byte stores and reads it back transposed.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include "gqa_decode.h"

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t uint4_t __attribute__((ext_vector_type(4)));

constexpr int kTile = 32;        // tokens per wave iteration (two 16-token MFMA row blocks)
constexpr int kWaves = 4;        // waves per partition workgroup
constexpr int kRedStride = 20;   // floats per (wave, d) row of the cross-wave buffer
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
};

// ------------------------------------------------------------ parameters --

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  const int32_t* block_table;   // paged only
  const int32_t* ctx_lens;      // paged only
  float2* part_ml;              // [num_seqs, h_q, max_parts] (m in log2 units, l)
  float* part_o;                // [num_seqs, h_q, max_parts, d]
  int num_seqs;
  int h_q;
  int h_kv;
  int group;                    // G = h_q / h_kv
  int s_kv;                     // contiguous length
  int max_blocks;               // paged table width
  int bs_shift;                 // log2(block_size)
  int max_ctx;                  // clamp for ctx_lens
  int part_size;
  int v1_max_ctx;
  int max_parts;
  float c;                      // scale * log2(e)
};

template <bool PAGED>
__device__ __forceinline__ int seq_len(const Params& a, int s) {
  if constexpr (PAGED) {
    const int L = a.ctx_lens[s];
    return min(max(L, 0), a.max_ctx);
  } else {
    return a.s_kv;
  }
}

// Orders this wave's LDS stores before its later LDS loads (and vice versa):
// the asm is a compiler memory barrier and the wait retires the wave's
// outstanding LDS operations.  Each wave only touches its own LDS region, so
// no workgroup barrier is needed inside the token loop.
__device__ __forceinline__ void wave_lds_fence() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Token held in k-slot e (0..7) of lane group grp: two 16-token halves, four
// consecutive tokens each.  The same slot order feeds P^T and V^T.
__device__ __forceinline__ int slot_token(int grp, int e) {
  return (e & 4) * 4 + grp * 4 + (e & 3);
}

// ------------------------------------------------------ partition kernel --

template <class DT, int D, bool PAGED, int NW>
__global__ __launch_bounds__(NW * 64) void partition_kernel(Params a) {
  constexpr int KK = D / 32;        // MFMA steps over d for Q.K^T
  constexpr int NB = D / 16;        // 16-row blocks of O^T
  constexpr int VS = D + 8;         // uint16 per staged V row (pad spreads LDS banks)
  constexpr int CH = D / 8;         // 16-byte chunks per K/V row
  constexpr int RPI = 64 / CH;      // V rows per 16-byte load instruction
  constexpr int NIT = kTile / RPI;  // V load instructions per tile
  constexpr int V_LDS = NW * kTile * VS * 2;
  constexpr int RED_LDS = NW * D * kRedStride * 4;
  constexpr int LDS_BYTES = V_LDS > RED_LDS ? V_LDS : RED_LDS;
  static_assert(LDS_BYTES <= 64 * 1024, "workgroup LDS budget");
  __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];

  // ---- work item: blockIdx.x = (s * h_kv + j) * max_parts + p
  const int p = blockIdx.x % a.max_parts;
  const int sj = blockIdx.x / a.max_parts;
  const int j = sj % a.h_kv;
  const int s = sj / a.h_kv;
  const int L = seq_len<PAGED>(a, s);
  const bool split = L > a.v1_max_ctx;
  const int n_part = split ? (L + a.part_size - 1) / a.part_size : 1;
  if (p >= n_part) return;                       // uniform over the workgroup
  const int t0 = split ? p * a.part_size : 0;
  const int t1 = split ? min(t0 + a.part_size, L) : L;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int col = lane & 15;                     // head column / K row within a half
  const int grp = lane >> 4;                     // 16-lane group
  const int G = a.group;
  const int head0 = j * G;

  // ---- Q^T operand: lane holds q[head col][8 d of chunk kk*4+grp]; zero rows pad G to 16
  uint4_t qop[KK];
  {
    const bool live = col < G;
    const uint16_t* qrow = a.q + ((int64_t)s * a.h_q + head0 + (live ? col : 0)) * D;
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

  uint16_t* vt = reinterpret_cast<uint16_t*>(lds) + w * kTile * VS;
  const int32_t* trow = PAGED ? a.block_table + (int64_t)s * a.max_blocks : nullptr;
  const int64_t tok_stride = (int64_t)a.h_kv * D;   // elements between consecutive tokens
  const int bs_mask = (1 << a.bs_shift) - 1;

  for (int tb = t0 + w * kTile; tb < t1; tb += NW * kTile) {
    // element offset of the first row of each 16-token half (tiles are 16-aligned,
    // block_size >= 16, so a half never straddles two physical blocks)
    int64_t base[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int th = tb + 16 * hb;
      if constexpr (PAGED) {
        const int32_t blk = th < t1 ? trow[th >> a.bs_shift] : 0;
        base[hb] = ((((int64_t)blk << a.bs_shift) + (th & bs_mask)) * a.h_kv + j) * D;
      } else {
        base[hb] = (((int64_t)s * a.s_kv + th) * a.h_kv + j) * D;
      }
    }

    // ---- issue all global loads of the tile first
    uint4_t vreg[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int r = it * RPI + lane / CH;
      const int c = lane % CH;
      vreg[it] = (tb + r < t1)
          ? *reinterpret_cast<const uint4_t*>(a.v + base[r >> 4] + (r & 15) * tok_stride + c * 8)
          : uint4_t{0u, 0u, 0u, 0u};
    }
    uint4_t kop[2][KK];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const bool ok = tb + 16 * hb + col < t1;
      const uint16_t* krow = a.k + base[hb] + col * tok_stride;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        kop[hb][kk] = ok ? *reinterpret_cast<const uint4_t*>(krow + 8 * (kk * 4 + grp))
                         : uint4_t{0u, 0u, 0u, 0u};
    }

    // ---- stage V (row-major, padded rows)
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int r = it * RPI + lane / CH;
      const int c = lane % CH;
      *reinterpret_cast<uint4_t*>(vt + r * VS + c * 8) = vreg[it];
    }

    // ---- scores S^T = K . Q^T
    float4_t sc[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      sc[hb] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) sc[hb] = DT::mfma(kop[hb][kk], qop[kk], sc[hb]);
    }

    // ---- online softmax (base 2); lane holds tokens slot_token(grp, e) of head col
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

    // ---- O^T += V^T . P^T, V^T read transposed from the staged tile
    wave_lds_fence();
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      uint32_t vv[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const uint32_t lo = vt[slot_token(grp, 2 * e2) * VS + 16 * nb + col];
        const uint32_t hi = vt[slot_token(grp, 2 * e2 + 1) * VS + 16 * nb + col];
        vv[e2] = lo | (hi << 16);
      }
      const uint4_t vop{vv[0], vv[1], vv[2], vv[3]};
      acc[nb] *= alpha;
      acc[nb] = DT::mfma(vop, phi4, acc[nb]);
      acc[nb] = DT::mfma(vop, plo4, acc[nb]);
    }
    wave_lds_fence();
  }

  // ---- merge the NW waves in LDS: red[(w*D + d)*kRedStride + head], with
  //      columns 16..19 of rows 0..3 holding m and of rows 4..7 holding l
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      red[(w * D + 16 * nb + 4 * grp + r) * kRedStride + col] = acc[nb][r];
  if (grp == 0) {
    red[(w * D + (col >> 2)) * kRedStride + 16 + (col & 3)] = m_run;
    red[(w * D + 4 + (col >> 2)) * kRedStride + 16 + (col & 3)] = l_run;
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < G * CH; idx += NW * 64) {
    const int g = idx / CH;
    const int d0 = (idx % CH) * 8;
    float mw[NW];
    float M = -INFINITY;
#pragma unroll
    for (int u = 0; u < NW; ++u) {
      mw[u] = red[(u * D + (g >> 2)) * kRedStride + 16 + (g & 3)];
      M = fmaxf(M, mw[u]);
    }
    float lsum = 0.f;
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < NW; ++u) {
      if (mw[u] == -INFINITY) continue;          // a wave that saw no token
      const float aw = __builtin_amdgcn_exp2f(mw[u] - M);
      lsum += aw * red[(u * D + 4 + (g >> 2)) * kRedStride + 16 + (g & 3)];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] += aw * red[(u * D + d0 + e) * kRedStride + g];
    }
    const int64_t row = (int64_t)s * a.h_q + head0 + g;
    if (!split) {
      uint32_t packed[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const uint32_t lo = L > 0 ? DT::narrow(o[2 * e2] / lsum) : 0u;
        const uint32_t hi = L > 0 ? DT::narrow(o[2 * e2 + 1] / lsum) : 0u;
        packed[e2] = lo | (hi << 16);
      }
      *reinterpret_cast<uint4_t*>(a.out + row * D + d0) =
          uint4_t{packed[0], packed[1], packed[2], packed[3]};
    } else {
      float* dst = a.part_o + (row * a.max_parts + p) * D + d0;
      *reinterpret_cast<float4_t*>(dst) = float4_t{o[0], o[1], o[2], o[3]};
      *reinterpret_cast<float4_t*>(dst + 4) = float4_t{o[4], o[5], o[6], o[7]};
      if (d0 == 0) a.part_ml[row * a.max_parts + p] = make_float2(M, lsum);
    }
  }
}

// ---------------------------------------------------------- merge kernel --

template <class DT, int D, bool PAGED>
__global__ __launch_bounds__(256) void merge_kernel(Params a) {
  constexpr int E = D / 64;                       // output elements per lane
  const int lane = threadIdx.x & 63;
  const int heads4 = (a.h_q + 3) >> 2;
  const int s = blockIdx.x / heads4;
  const int i = (blockIdx.x % heads4) * 4 + (threadIdx.x >> 6);
  if (i >= a.h_q) return;                         // no barriers below: per-wave exit is safe
  const int L = seq_len<PAGED>(a, s);
  if (L <= a.v1_max_ctx) return;                  // written by the partition kernel
  const int n = (L + a.part_size - 1) / a.part_size;
  const int64_t row = (int64_t)s * a.h_q + i;
  const float2* ml = a.part_ml + row * a.max_parts;
  const float* po = a.part_o + row * a.max_parts * D + lane * E;

  float M = -INFINITY;
  for (int pp = lane; pp < n; pp += 64) M = fmaxf(M, ml[pp].x);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));

  // fixed partition order: the result does not depend on scheduling
  float lsum = 0.f;
  float o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;
  for (int pp = 0; pp < n; ++pp) {
    const float2 t = ml[pp];
    const float wgt = __builtin_amdgcn_exp2f(t.x - M);
    lsum += wgt * t.y;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] += wgt * po[(int64_t)pp * D + e];
  }
  uint16_t* dst = a.out + row * D + lane * E;
#pragma unroll
  for (int e = 0; e < E; ++e) dst[e] = static_cast<uint16_t>(DT::narrow(o[e] / lsum));
}

// ------------------------------------------------------------------ host --

constexpr int32_t kDefaultPartition = 1024;
constexpr int32_t kDefaultV1Max = 1024;

struct Problem {
  bool paged;
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
};

bool aligned(const void* ptr, uintptr_t n) { return (reinterpret_cast<uintptr_t>(ptr) & (n - 1)) == 0; }

gqa_status_t resolve_policy(const gqa_policy_t* in, gqa_policy_t* out) {
  if (in == nullptr)
    gqa_policy_default(out);
  else
    *out = *in;
  if (out->partition_size < kTile || out->partition_size > (1 << 20) ||
      out->partition_size % kTile != 0 || out->v1_max_ctx < 0 || out->phases < 0 ||
      out->phases > 3 || out->reserved != 0)
    return GQA_ERR_BAD_POLICY;
  if (out->phases == 0) out->phases = 3;
  return GQA_OK;
}

int parts_for(int max_ctx, const gqa_policy_t& pol) {
  if (max_ctx <= pol.v1_max_ctx) return 1;
  return (int)(((int64_t)max_ctx + pol.partition_size - 1) / pol.partition_size);
}

size_t workspace_for(int num_seqs, int h_q, int d, int max_ctx, const gqa_policy_t& pol) {
  if (max_ctx <= pol.v1_max_ctx) return 0;
  const size_t rows = (size_t)num_seqs * (size_t)h_q * (size_t)parts_for(max_ctx, pol);
  const size_t ml = (rows * sizeof(float2) + 255) & ~(size_t)255;
  return ml + rows * (size_t)d * sizeof(float);
}

template <class DT, int D, bool PAGED>
gqa_status_t launch_typed(const Params& prm, int grid_parts, int grid_merge, int phases,
                          hipStream_t stream) {
  Params local = prm;
  void* args[] = {&local};
  if ((phases & 1) && grid_parts > 0) {
    if (hipLaunchKernel(reinterpret_cast<const void*>(&partition_kernel<DT, D, PAGED, kWaves>),
                        dim3(grid_parts), dim3(kWaves * 64), args, 0, stream) != hipSuccess)
      return GQA_ERR_LAUNCH;
  }
  if ((phases & 2) && grid_merge > 0) {
    if (hipLaunchKernel(reinterpret_cast<const void*>(&merge_kernel<DT, D, PAGED>),
                        dim3(grid_merge), dim3(256), args, 0, stream) != hipSuccess)
      return GQA_ERR_LAUNCH;
  }
  return GQA_OK;
}

template <class DT>
gqa_status_t launch_dtype(const Problem& pb, const Params& prm, int gp, int gm, int ph,
                          hipStream_t st) {
  if (pb.d == 64)
    return pb.paged ? launch_typed<DT, 64, true>(prm, gp, gm, ph, st)
                    : launch_typed<DT, 64, false>(prm, gp, gm, ph, st);
  return pb.paged ? launch_typed<DT, 128, true>(prm, gp, gm, ph, st)
                  : launch_typed<DT, 128, false>(prm, gp, gm, ph, st);
}

gqa_status_t run(const Problem& pb) {
  // ---- sizes, shapes, support (no HIP call before every check has passed)
  if (pb.num_seqs < 0 || pb.h_q <= 0 || pb.h_kv <= 0 || pb.h_q % pb.h_kv != 0)
    return GQA_ERR_BAD_SHAPE;
  if (pb.paged ? (pb.max_blocks <= 0) : (pb.s_kv < 0)) return GQA_ERR_BAD_SHAPE;
  if (pb.dtype != GQA_F16 && pb.dtype != GQA_BF16) return GQA_ERR_UNSUPPORTED;
  if (pb.d != 64 && pb.d != 128) return GQA_ERR_UNSUPPORTED;
  const int G = pb.h_q / pb.h_kv;
  if (G > 16) return GQA_ERR_UNSUPPORTED;
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
  const int max_parts = parts_for(max_ctx, pol);
  const int64_t grid_parts = (int64_t)max_parts * pb.h_kv * pb.num_seqs;
  const int64_t grid_merge = (max_ctx > pol.v1_max_ctx) ? (int64_t)((pb.h_q + 3) / 4) * pb.num_seqs : 0;
  if (grid_parts > INT32_MAX || grid_merge > INT32_MAX) return GQA_ERR_BAD_SHAPE;
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
  const size_t need = workspace_for(pb.num_seqs, pb.h_q, pb.d, max_ctx, pol);
  if (need > 0) {
    if (!pb.ws || pb.ws_bytes < need) return GQA_ERR_WORKSPACE;
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
  const size_t rows = (size_t)pb.num_seqs * pb.h_q * max_parts;
  prm.part_ml = need ? static_cast<float2*>(pb.ws) : nullptr;
  prm.part_o = need ? reinterpret_cast<float*>(static_cast<char*>(pb.ws) +
                                               ((rows * sizeof(float2) + 255) & ~(size_t)255))
                    : nullptr;
  prm.num_seqs = pb.num_seqs;
  prm.h_q = pb.h_q;
  prm.h_kv = pb.h_kv;
  prm.group = G;
  prm.s_kv = pb.s_kv;
  prm.max_blocks = pb.max_blocks;
  prm.bs_shift = bs_shift;
  prm.max_ctx = max_ctx;
  prm.part_size = pol.partition_size;
  prm.v1_max_ctx = pol.v1_max_ctx;
  prm.max_parts = max_parts;
  prm.c = pb.scale * kLog2e;
  hipStream_t st = static_cast<hipStream_t>(pb.stream);
  if (pb.dtype == GQA_F16)
    return launch_dtype<F16>(pb, prm, (int)grid_parts, (int)grid_merge, pol.phases, st);
  return launch_dtype<BF16>(pb, prm, (int)grid_parts, (int)grid_merge, pol.phases, st);
}

}  // namespace

extern "C" {

void gqa_policy_default(gqa_policy_t* p) {
  if (!p) return;
  p->partition_size = kDefaultPartition;
  p->v1_max_ctx = kDefaultV1Max;
  p->phases = 0;
  p->reserved = 0;
}

void gqa_policy_pages(gqa_policy_t* p) {
  if (!p) return;
  p->partition_size = 512;
  p->v1_max_ctx = 8192;
  p->phases = 0;
  p->reserved = 0;
}

size_t gqa_decode_workspace_size(int num_seqs, int h_q, int d_head, int max_ctx,
                                 const gqa_policy_t* policy) {
  gqa_policy_t pol;
  if (resolve_policy(policy, &pol) != GQA_OK) return 0;
  if (num_seqs < 0 || h_q <= 0 || d_head <= 0 || max_ctx < 0) return 0;
  return workspace_for(num_seqs, h_q, d_head, max_ctx, pol);
}

gqa_status_t gqa_decode(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_table, const int32_t* ctx_lens, void* out,
                        int num_seqs, int max_blocks_per_seq, int h_q, int h_kv,
                        int d_head, int block_size, float scale, gqa_dtype_t dtype,
                        void* workspace, size_t workspace_bytes,
                        const gqa_policy_t* policy, void* stream) {
  Problem pb{};
  pb.paged = true;
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

gqa_status_t gqa_decode_contiguous(const void* q, const void* k, const void* v, void* out,
                                   int num_seqs, int s_kv, int h_q, int h_kv, int d_head,
                                   float scale, gqa_dtype_t dtype,
                                   void* workspace, size_t workspace_bytes,
                                   const gqa_policy_t* policy, void* stream) {
  Problem pb{};
  pb.paged = false;
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

const char* gqa_status_string(gqa_status_t status) {
  switch (status) {
    case GQA_OK: return "GQA_OK: success";
    case GQA_ERR_NULL_PTR: return "GQA_ERR_NULL_PTR: a required pointer is NULL";
    case GQA_ERR_BAD_SHAPE: return "GQA_ERR_BAD_SHAPE: invalid or inconsistent sizes";
    case GQA_ERR_UNSUPPORTED: return "GQA_ERR_UNSUPPORTED: d_head, group size, block size or dtype not supported";
    case GQA_ERR_MISALIGNED: return "GQA_ERR_MISALIGNED: pointer alignment requirement not met";
    case GQA_ERR_WORKSPACE: return "GQA_ERR_WORKSPACE: workspace missing or too small";
    case GQA_ERR_BAD_POLICY: return "GQA_ERR_BAD_POLICY: policy fields out of range";
    case GQA_ERR_BAD_SCALE: return "GQA_ERR_BAD_SCALE: scale is not finite";
    case GQA_ERR_LAUNCH: return "GQA_ERR_LAUNCH: kernel launch failed";
  }
  return "unknown gqa_status_t";
}

}  // extern "C"
