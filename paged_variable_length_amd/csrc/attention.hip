// HIP kernels and launchers of libpagedattn.so, written for gfx950 (MI355X, CDNA4).
//
// Kernels
//   reshape_and_cache_kernel  copy of new K/V rows into their page slots (HBM-bound copy)
//   decode_kernel             split-K decode attention, one workgroup per decode task
//   meta_attn_kernel          one grid over a mixed, load-sorted task table: each workgroup
//                             reads its task's kind and runs the decode or the prefill body
//   combine_kernel            log-sum-exp merge of split partials into `out`
//
// Decode body (HBM-bound). A task is (sequence, kv head, key range). Its four waves take
// interleaved chunks of the key range. Scores S = K Q^T come from 16x16x32 bf16 MFMAs whose
// 16 columns are the G query heads of the kv head (zero-padded to 16), so every K/V page is
// read once for all heads of its group. K rows are loaded straight into the MFMA operand
// layout; V rows are loaded 16 bytes per lane along D and rearranged in registers, so the
// value product O^T = V^T P^T consumes them without an LDS round trip and each lane ends up
// owning one head's slice of D. Online softmax in base 2, per head; the four waves merge
// through LDS at the end and write either the output row or an fp32 partial.
//
// Prefill body (MFMA-bound). A task is (sequence, query head, up to 128 query rows, key
// range). 64-key K/V tiles are gathered through the block table into double-buffered LDS;
// each wave owns 32 query rows, computes S^T = K Q^T and O^T += V^T P^T with 32x32x16 bf16
// MFMAs, and applies the causal mask only on tiles that cross the diagonal.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;  // 4 waves of 64
constexpr float kLog2e = 1.4426950408889634f;

struct AttnArgs {
  const void* q;
  const void* k_pages;
  const void* v_pages;
  const int32_t* block_table;
  const int32_t* cu_seqlens;    // nullptr: one query row per sequence, token index = seq
  const int32_t* context_lens;  // used by prefill tasks (cached prefix length)
  const pa_task* tasks;
  float* ws_acc;                // [num_partials, D]
  float* ws_ml;                 // [num_partials, 2] (running max in log2 units, sum)
  void* out;
  int32_t max_blocks;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t bs_shift;
  int32_t num_tasks;
  float scale_log2;             // softmax scale * log2(e)
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Low (k even) or high (k odd) bf16 halves of two dwords, packed as (a_half, b_half).
__device__ __forceinline__ uint32_t pair_half(uint32_t a, uint32_t b, int odd) {
  return odd ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
}

// ------------------------------------------------------------------------------------------
// Decode body, bf16. Lane map inside a wave: i16 = lane & 15, g4 = lane >> 4.
//   QK  (16x16x32): A = K tile [16 tokens x 32 d], B = Q^T [32 d x 16 heads]
//                   lane supplies token/head i16 and d = 32*ks + 8*g4 + 0..7.
//   S   C-layout:   lane holds S[token 4*g4 + r][head i16], r = 0..3.
//   PV  (16x16x32): A = V^T [16 d-rows x 32 tokens], B = P^T [32 tokens x 16 heads]
//                   k-slot (g4, e) <-> token 4*g4 + e (e < 4, first 16-token tile) or
//                   16 + 4*g4 + e - 4 (second tile); d-row i16 of block n <-> d = VEC*i16 + n.
//   O   C-layout:   acc[n][r] = O[head i16][d = VEC*(4*g4 + r) + n].
// ------------------------------------------------------------------------------------------
template <int D>
struct DecodeVRaw;
template <>
struct DecodeVRaw<128> {
  typedef u32x4 type;  // 8 bf16 along D
};
template <>
struct DecodeVRaw<64> {
  typedef u32x2 type;  // 4 bf16 along D
};

template <int D>
__device__ __forceinline__ void decode_merge_and_store(const AttnArgs& a, const pa_task& t,
                                                       int tok, int G, float m, float l,
                                                       const f32x4* acc, float* smem,
                                                       bool out_bf16) {
  constexpr int VEC = D / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g4 = lane >> 4;
  l += wave_shfl_xor(l, 16);
  l += wave_shfl_xor(l, 32);
  float* sm_m = smem;              // [4][16]
  float* sm_l = smem + 64;         // [4][16]
  float* sm_acc = smem + 128;      // [4][16][D]
  if (g4 == 0) {
    sm_m[wave * 16 + i16] = m;
    sm_l[wave * 16 + i16] = l;
  }
  if (i16 < G) {
#pragma unroll
    for (int n = 0; n < VEC; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) sm_acc[(wave * 16 + i16) * D + VEC * (4 * g4 + r) + n] = acc[n][r];
  }
  __syncthreads();
  const int hq0 = t.head * G;
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int h = idx / D, d = idx - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w * 16 + h]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float wt = fast_exp2(sm_m[w * 16 + h] - M);
      L += wt * sm_l[w * 16 + h];
      A += wt * sm_acc[(w * 16 + h) * D + d];
    }
    if (t.partial < 0) {
      const size_t o = (static_cast<size_t>(tok) * a.num_q_heads + hq0 + h) * D + d;
      const float v = A / L;
      if (out_bf16)
        static_cast<__bf16*>(a.out)[o] = static_cast<__bf16>(v);
      else
        static_cast<float*>(a.out)[o] = v;
    } else {
      const size_t row = static_cast<size_t>(t.partial) + h;
      a.ws_acc[row * D + d] = A;
      if (d == 0) {
        a.ws_ml[2 * row] = M;
        a.ws_ml[2 * row + 1] = L;
      }
    }
  }
}

template <int D>
__device__ void decode_task_bf16(const AttnArgs& a, const pa_task& t, float* smem) {
  constexpr int KS = D / 32;
  constexpr int VEC = D / 16;
  typedef typename DecodeVRaw<D>::type VRaw;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g4 = lane >> 4;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int s = t.seq, kvh = t.head;
  const int tok = a.cu_seqlens ? a.cu_seqlens[s] : s;
  const int bs = a.block_size;

  bf16x8 qf[KS];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         (static_cast<size_t>(tok) * a.num_q_heads + kvh * G + i16) * D + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (i16 < G) v = *reinterpret_cast<const u32x4*>(qp + 32 * ks);
      qf[ks] = as_bf16x8(v);
    }
  }
  const size_t head_stride = static_cast<size_t>(bs) * D;
  const size_t block_stride = static_cast<size_t>(a.num_kv_heads) * head_stride;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k_pages) + kvh * head_stride;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v_pages) + kvh * head_stride;
  const int32_t* bt = a.block_table + static_cast<size_t>(s) * a.max_blocks;
  const float c = a.scale_log2;

  f32x4 acc[VEC];
#pragma unroll
  for (int n = 0; n < VEC; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  const int kv0 = t.kv0, kv1 = t.kv1;
  const int nchunks = (kv1 - kv0 + 31) >> 5;
  for (int ch = wave; ch < nchunks; ch += 4) {
    const int cs = kv0 + 32 * ch;
    size_t off[2];
    bool tv[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int ts = cs + 16 * tt;
      tv[tt] = ts < kv1;
      const int blk = tv[tt] ? bt[ts >> a.bs_shift] : 0;
      off[tt] = static_cast<size_t>(blk) * block_stride + static_cast<size_t>(ts & (bs - 1)) * D;
    }
    bf16x8 kf[2][KS];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (tv[tt])
          v = *reinterpret_cast<const u32x4*>(kbase + off[tt] + i16 * D + 32 * ks + 8 * g4);
        kf[tt][ks] = as_bf16x8(v);
      }
    VRaw vr[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int tt = e >> 2;
      VRaw v = {};
      if (tv[tt])
        v = *reinterpret_cast<const VRaw*>(vbase + off[tt] + (4 * g4 + (e & 3)) * D + VEC * i16);
      vr[e] = v;
    }
    f32x4 sc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      sc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        sc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[tt][ks], qf[ks], sc[tt], 0, 0, 0);
    }
    if (cs + 32 > kv1) {
      // tail chunk: keys past kv1 get no weight, and their (possibly non-finite) values are
      // replaced by zeros so that 0 * value stays 0 in the value product
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = cs + 16 * (e >> 2) + 4 * g4 + (e & 3);
        if (key >= kv1) {
          sc[e >> 2][e & 3] = -INFINITY;
          vr[e] = VRaw{};
        }
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mx = fmaxf(mx, wave_shfl_xor(mx, 16));
    mx = fmaxf(mx, wave_shfl_xor(mx, 32));
    const float mnew = fmaxf(m, mx * c);
    const float muse = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = fast_exp2(m - muse);
    float p[8];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = fast_exp2(fmaf(sc[e >> 2][e & 3], c, -muse));
      psum += p[e];
    }
    l = l * alpha + psum;
    m = mnew;
#pragma unroll
    for (int n = 0; n < VEC; ++n) acc[n] *= alpha;
    u32x4 pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                pack_bf16x2(p[6], p[7])};
    const bf16x8 pf = as_bf16x8(pw);
#pragma unroll
    for (int n = 0; n < VEC; ++n) {
      u32x4 vw;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        vw[qd] = pair_half(vr[2 * qd][n >> 1], vr[2 * qd + 1][n >> 1], n & 1);
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vw), pf, acc[n], 0, 0, 0);
    }
  }
  decode_merge_and_store<D>(a, t, tok, G, m, l, acc, smem, true);
}

// ------------------------------------------------------------------------------------------
// Decode body, fp32 inputs, 16x16x4 fp32 MFMAs, 16-token chunks.
//   QK: A = K [16 tokens x 4 d], B = Q^T; lane supplies d = 16*kq + 4*g4 + u at k-step (kq, u).
//   PV: k-step r uses token 4*g4 + r; A = V^T with d-row i16 of block n <-> d = VEC*i16 + n.
//   O:  acc[n][r] = O[head i16][d = VEC*(4*g4 + r) + n] (same map as the bf16 body).
// ------------------------------------------------------------------------------------------
template <int D>
__device__ void decode_task_f32(const AttnArgs& a, const pa_task& t, float* smem) {
  constexpr int KQ = D / 16;
  constexpr int VEC = D / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g4 = lane >> 4;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int s = t.seq, kvh = t.head;
  const int tok = a.cu_seqlens ? a.cu_seqlens[s] : s;
  const int bs = a.block_size;

  f32x4 qf[KQ];
  {
    const float* qp = static_cast<const float*>(a.q) +
                      (static_cast<size_t>(tok) * a.num_q_heads + kvh * G + i16) * D + 4 * g4;
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq) {
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (i16 < G) v = *reinterpret_cast<const f32x4*>(qp + 16 * kq);
      qf[kq] = v;
    }
  }
  const size_t head_stride = static_cast<size_t>(bs) * D;
  const size_t block_stride = static_cast<size_t>(a.num_kv_heads) * head_stride;
  const float* kbase = static_cast<const float*>(a.k_pages) + kvh * head_stride;
  const float* vbase = static_cast<const float*>(a.v_pages) + kvh * head_stride;
  const int32_t* bt = a.block_table + static_cast<size_t>(s) * a.max_blocks;
  const float c = a.scale_log2;

  f32x4 acc[VEC];
#pragma unroll
  for (int n = 0; n < VEC; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;
  const int kv0 = t.kv0, kv1 = t.kv1;
  const int nchunks = (kv1 - kv0 + 15) >> 4;
  for (int ch = wave; ch < nchunks; ch += 4) {
    const int ts = kv0 + 16 * ch;
    const int blk = bt[ts >> a.bs_shift];
    const size_t off = static_cast<size_t>(blk) * block_stride + static_cast<size_t>(ts & (bs - 1)) * D;
    f32x4 kf[KQ];
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq)
      kf[kq] = *reinterpret_cast<const f32x4*>(kbase + off + i16 * D + 16 * kq + 4 * g4);
    float vr[4][VEC];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int v4 = 0; v4 < VEC; v4 += 4) {
        const f32x4 v =
            *reinterpret_cast<const f32x4*>(vbase + off + (4 * g4 + r) * D + VEC * i16 + v4);
        vr[r][v4] = v[0];
        vr[r][v4 + 1] = v[1];
        vr[r][v4 + 2] = v[2];
        vr[r][v4 + 3] = v[3];
      }
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        sc = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[kq][u], qf[kq][u], sc, 0, 0, 0);
    if (ts + 16 > kv1) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (ts + 4 * g4 + r >= kv1) {
          sc[r] = -INFINITY;
#pragma unroll
          for (int n = 0; n < VEC; ++n) vr[r][n] = 0.f;
        }
    }
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = fmaxf(mx, wave_shfl_xor(mx, 16));
    mx = fmaxf(mx, wave_shfl_xor(mx, 32));
    const float mnew = fmaxf(m, mx * c);
    const float muse = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = fast_exp2(m - muse);
    float p[4];
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = fast_exp2(fmaf(sc[r], c, -muse));
      psum += p[r];
    }
    l = l * alpha + psum;
    m = mnew;
#pragma unroll
    for (int n = 0; n < VEC; ++n) acc[n] *= alpha;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int n = 0; n < VEC; ++n)
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(vr[r][n], p[r], acc[n], 0, 0, 0);
  }
  decode_merge_and_store<D>(a, t, tok, G, m, l, acc, smem, false);
}

// ------------------------------------------------------------------------------------------
// Prefill body, bf16. Lane map inside a wave: i32 = lane & 31, g2 = lane >> 5.
//   QK (32x32x16): A = K [32 keys x 16 d], B = Q^T [16 d x 32 rows];
//                  lane supplies key/row i32 and d = 16*ks + 8*g2 + 0..7.
//   S^T C-layout:  reg r of key block kb = S[row i32][key 32*kb + 8*(r/4) + 4*g2 + r%4].
//   PV (32x32x16): A = V^T [32 d-rows x 16 keys], B = P^T [16 keys x 32 rows];
//                  k-step kk, slot (g2, e) <-> key 16*kk + 8*(e/4) + 4*g2 + e%4,
//                  d-row i of block n <-> d = 32*n + i.
//   O^T C-layout:  acc[n] reg r = O[row i32][d = 32*n + 8*(r/4) + 4*g2 + r%4].
// K/V tiles reach LDS by direct global->LDS loads (16 bytes per lane, 1 KiB per wave
// instruction). Rows are stored unpadded with the 16-byte chunks of key row k permuted by
// XOR with swz(k), so the K reads (eight consecutive keys, one chunk) and the transposed V
// reads (four keys, two neighbouring chunks) spread over distinct banks.
// V^T operands come from ds_read_b64_tr_b16: within each 16-lane group, lane j = 4r + c
// returns element c of the 8-byte segments addressed by lanes r, 4+r, 8+r, 12+r. With lane k
// of the group addressing key kbase + k/4, d = d0 + 4*(k%4), lane j receives the four keys
// kbase .. kbase+3 at d = d0 + j -- a column of V, as the MFMA operand needs.
// ------------------------------------------------------------------------------------------
template <int D>
struct PrefillCfg {
  static constexpr int kTile = 64;                                  // keys per LDS tile
  static constexpr int kRowBytes = D * 2;                           // one bf16 key row
  static constexpr int kChunks = D / 8;                             // 16-byte chunks per row
  static constexpr int kTileBytes = kTile * kRowBytes;
  static constexpr int kKeysPerLoad = 1024 / kRowBytes;             // keys per wave load
  static constexpr int kLoadsPerWave = kTileBytes / 1024 / 4;       // per tensor per tile
  static constexpr size_t kSmemBytes = 4 * static_cast<size_t>(kTileBytes);  // K,V x 2 bufs
};

__device__ __forceinline__ int lds_swz(int key) { return ((key & 3) << 1) | ((key >> 2) & 1); }

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <int D>
__device__ void prefill_task(const AttnArgs& a, const pa_task& t, char* smem) {
  typedef PrefillCfg<D> C;
  constexpr int KS = D / 16;   // k-steps of the QK product
  constexpr int NB = D / 32;   // 32-row d blocks of O^T
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i32 = lane & 31, g2 = lane >> 5;
  const int s = t.seq, h = t.head;
  const int cu0 = a.cu_seqlens[s];
  const int ql = a.cu_seqlens[s + 1] - cu0;
  const int prefix = a.context_lens[s] - ql;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int kvh = h / G;
  const int bs = a.block_size;
  const int r0 = t.q_row0, rows = t.q_rows;
  const int kv0 = t.kv0, kv1 = t.kv1;
  const int qi = r0 + 32 * wave + i32;              // this lane's query row (sequence-relative)
  const bool row_ok = qi < r0 + rows;
  const bool wave_active = 32 * wave < rows;
  const int wave_pos_lo = prefix + r0 + 32 * wave;  // position of the wave's first row
  const float c = a.scale_log2;

  bf16x8 qf[KS];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         (static_cast<size_t>(cu0 + qi) * a.num_q_heads + h) * D + 8 * g2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row_ok) v = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
      qf[ks] = as_bf16x8(v);
    }
  }

  const size_t head_stride = static_cast<size_t>(bs) * D;
  const size_t block_stride = static_cast<size_t>(a.num_kv_heads) * head_stride;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k_pages) + kvh * head_stride;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v_pages) + kvh * head_stride;
  const int32_t* bt = a.block_table + static_cast<size_t>(s) * a.max_blocks;
  char* sk = smem;                          // [2][kTileBytes]
  char* sv = smem + 2 * C::kTileBytes;      // [2][kTileBytes]

  // Each wave moves kLoadsPerWave 1 KiB pieces of the K tile and of the V tile. Keys past kv1
  // are read from key kv1-1 instead (valid memory, finite values); they are masked below.
  auto issue_tile = [&](int ts, int buf) {
#pragma unroll
    for (int i = 0; i < C::kLoadsPerWave; ++i) {
      const int piece = wave * C::kLoadsPerWave + i;
      const int key = piece * C::kKeysPerLoad + lane / C::kChunks;
      const int chunk = (lane % C::kChunks) ^ lds_swz(key);
      const int kabs = min(ts + key, kv1 - 1);
      const int blk = bt[kabs >> a.bs_shift];
      const size_t o = static_cast<size_t>(blk) * block_stride +
                       static_cast<size_t>(kabs & (bs - 1)) * D + chunk * 8;
      __builtin_amdgcn_global_load_lds(
          kbase + o, (__attribute__((address_space(3))) void*)(sk + buf * C::kTileBytes + piece * 1024),
          16, 0, 0);
      __builtin_amdgcn_global_load_lds(
          vbase + o, (__attribute__((address_space(3))) void*)(sv + buf * C::kTileBytes + piece * 1024),
          16, 0, 0);
    }
  };

  f32x16 acc[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[n][r] = 0.f;
  float m = -INFINITY, l = 0.f;

  // V^T operand addressing (see the header comment): group gq = lane / 16, j = lane % 16
  const int gq = lane >> 4, jq = lane & 15;
  const int v_key_off = 4 * g2 + (jq >> 2);                 // + 16*kk (+ 8 for the 2nd read)
  const int v_d = 16 * (gq & 1) + 4 * (jq & 3);             // + 32*n
  const int v_byte_in_chunk = 8 * (jq & 1);

  const int ntiles = (kv1 - kv0 + C::kTile - 1) / C::kTile;
  issue_tile(kv0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int ts = kv0 + it * C::kTile;
    const int buf = it & 1;
    if (it + 1 < ntiles) issue_tile(ts + C::kTile, buf ^ 1);
    // skip tiles whose every key lies after every row of this wave
    if (wave_active && ts <= wave_pos_lo + 31) {
      const char* kt = sk + buf * C::kTileBytes;
      const char* vt = sv + buf * C::kTileBytes;
      f32x16 sc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[kb][r] = 0.f;
        const int key = kb * 32 + i32;
        const char* krow = kt + key * C::kRowBytes;
        const int sw = lds_swz(key);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const u32x4 kw = *reinterpret_cast<const u32x4*>(krow + (((2 * ks + g2) ^ sw) << 4));
          sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kw), qf[ks], sc[kb], 0, 0, 0);
        }
      }
      if (ts + C::kTile - 1 > wave_pos_lo || ts + C::kTile > kv1) {
        const int pos = prefix + qi;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = ts + kb * 32 + 8 * (r >> 2) + 4 * g2 + (r & 3);
            if (key >= kv1 || key > pos) sc[kb][r] = -INFINITY;
          }
      }
      float mx = sc[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
      mx = fmaxf(mx, wave_shfl_xor(mx, 32)) * c;
      // Lazy rescale: keep the running max while the tile's max exceeds it by at most 8
      // (weights stay <= 2^8); numerator and denominator share the same reference, so the
      // result is unchanged.
      if (__builtin_amdgcn_ballot_w64(mx > m + 8.f) != 0) {
        const float mnew = fmaxf(m, mx);
        const float alpha = mnew == -INFINITY ? 1.f : fast_exp2(m - mnew);
        l *= alpha;
#pragma unroll
        for (int n = 0; n < NB; ++n) acc[n] *= alpha;
        m = mnew;
      }
      const float muse = m == -INFINITY ? 0.f : m;
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sc[kb][r] = fast_exp2(fmaf(sc[kb][r], c, -muse));
          psum += sc[kb][r];
        }
      l += psum;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int kb = kk >> 1, rb = 8 * (kk & 1);
        u32x4 pw = {pack_bf16x2(sc[kb][rb + 0], sc[kb][rb + 1]),
                    pack_bf16x2(sc[kb][rb + 2], sc[kb][rb + 3]),
                    pack_bf16x2(sc[kb][rb + 4], sc[kb][rb + 5]),
                    pack_bf16x2(sc[kb][rb + 6], sc[kb][rb + 7])};
        const bf16x8 pf = as_bf16x8(pw);
        const int key1 = 16 * kk + v_key_off;
        const int key2 = key1 + 8;
        const char* vrow1 = vt + key1 * C::kRowBytes + v_byte_in_chunk;
        const char* vrow2 = vt + key2 * C::kRowBytes + v_byte_in_chunk;
        const int sw1 = lds_swz(key1), sw2 = lds_swz(key2);
#pragma unroll
        for (int n = 0; n < NB; ++n) {
          const int chunk = (32 * n + v_d) >> 3;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(vrow1 + ((chunk ^ sw1) << 4)));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(vrow2 + ((chunk ^ sw2) << 4)));
          const u32x4 vw = {__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                            __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]};
          acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vw), pf, acc[n], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  l += wave_shfl_xor(l, 32);
  if (!row_ok) return;
  if (t.partial < 0) {
    const float inv = 1.f / l;
    __bf16* orow = static_cast<__bf16*>(a.out) +
                   (static_cast<size_t>(cu0 + qi) * a.num_q_heads + h) * D;
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const int d0 = 32 * n + 8 * rb + 4 * g2;
        *reinterpret_cast<u32x2*>(orow + d0) =
            u32x2{pack_bf16x2(acc[n][4 * rb] * inv, acc[n][4 * rb + 1] * inv),
                  pack_bf16x2(acc[n][4 * rb + 2] * inv, acc[n][4 * rb + 3] * inv)};
      }
  } else {
    const size_t row = static_cast<size_t>(t.partial) + (qi - r0);
    float* prow = a.ws_acc + row * D;
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
        *reinterpret_cast<f32x4*>(prow + 32 * n + 8 * rb + 4 * g2) =
            f32x4{acc[n][4 * rb], acc[n][4 * rb + 1], acc[n][4 * rb + 2], acc[n][4 * rb + 3]};
    if (g2 == 0) {
      a.ws_ml[2 * row] = m;
      a.ws_ml[2 * row + 1] = l;
    }
  }
}

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup i runs on XCD i % 8).
// Within each full window of 64 consecutive workgroups, XCD x receives the 8 consecutive
// table entries 8x .. 8x+7, so neighbouring tasks (query heads that share one kv head's pages)
// meet in one L2. The load-sorted order changes only inside a window.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int base = bid & ~63;
  if (base + 64 > n) return bid;
  const int r = bid & 63;
  return base + (r & 7) * 8 + (r >> 3);
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void decode_kernel(AttnArgs a) {
  __shared__ float smem[128 + 4 * 16 * D];
  const pa_task t = a.tasks[blockIdx.x];
  if (t.kind != PA_TASK_DECODE) return;
  if constexpr (sizeof(T) == 2)
    decode_task_bf16<D>(a, t, smem);
  else
    decode_task_f32<D>(a, t, smem);
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void meta_attn_kernel(AttnArgs a) {
  constexpr size_t kPrefill = PrefillCfg<D>::kSmemBytes;
  constexpr size_t kDecode = (128 + 4 * 16 * D) * sizeof(float);
  __shared__ __attribute__((aligned(1024))) char smem[kPrefill > kDecode ? kPrefill : kDecode];
  const pa_task t = a.tasks[xcd_remap(blockIdx.x, a.num_tasks)];
  if (t.kind == PA_TASK_DECODE)
    decode_task_bf16<D>(a, t, reinterpret_cast<float*>(smem));
  else
    prefill_task<D>(a, t, smem);
}

// One workgroup per combine record; each wave merges one (row, head) at a time.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void combine_kernel(const pa_combine* combines,
                                                           const int32_t* cu_seqlens,
                                                           const float* ws_acc,
                                                           const float* ws_ml, T* out,
                                                           int32_t num_q_heads) {
  constexpr int PER = D / 64;
  const pa_combine cb = combines[blockIdx.x];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tok0 = (cu_seqlens ? cu_seqlens[cb.seq] : cb.seq) + cb.q_row0;
  const int R = cb.q_rows * cb.heads;
  for (int row = wave; row < R; row += 4) {
    const int i = row / cb.heads, j = row - i * cb.heads;
    float M = -INFINITY;
    for (int k = 0; k < cb.n_slots; ++k)
      M = fmaxf(M, ws_ml[2 * (static_cast<size_t>(cb.first_slot) + static_cast<size_t>(k) * R + row)]);
    float L = 0.f, acc[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) acc[u] = 0.f;
    for (int k = 0; k < cb.n_slots; ++k) {
      const size_t slot = static_cast<size_t>(cb.first_slot) + static_cast<size_t>(k) * R + row;
      const float w = fast_exp2(ws_ml[2 * slot] - M);
      L += w * ws_ml[2 * slot + 1];
#pragma unroll
      for (int u = 0; u < PER; ++u) acc[u] += w * ws_acc[slot * D + lane * PER + u];
    }
    const float inv = 1.f / L;
    T* orow = out + (static_cast<size_t>(tok0 + i) * num_q_heads + cb.head + j) * D + lane * PER;
#pragma unroll
    for (int u = 0; u < PER; ++u) orow[u] = static_cast<T>(acc[u] * inv);
  }
}

// One workgroup per packed token: find its sequence, then copy the token's K and V rows of
// every kv head (16 bytes per thread per step) into the page slot the block table assigns.
template <int ROW_BYTES>
__global__ __launch_bounds__(kThreads) void reshape_and_cache_kernel(
    const uint8_t* k_new, const uint8_t* v_new, uint8_t* k_pages, uint8_t* v_pages,
    const int32_t* block_table, int32_t max_blocks, const int32_t* cu_seqlens,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_kv_heads, int32_t block_size,
    int32_t bs_shift) {
  constexpr int CH = ROW_BYTES / 16;  // 16-byte chunks per (token, head) row
  const int t = blockIdx.x;
  int lo = 0, hi = num_seqs;  // cu[lo] <= t < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu_seqlens[mid] <= t) lo = mid; else hi = mid;
  }
  const int s = lo;
  const int qlen = cu_seqlens[s + 1] - cu_seqlens[s];
  const int pos = context_lens[s] - qlen + (t - cu_seqlens[s]);
  const int blk = block_table[static_cast<size_t>(s) * max_blocks + (pos >> bs_shift)];
  const int slot = pos & (block_size - 1);
  const int per_tensor = num_kv_heads * CH;
  for (int c = threadIdx.x; c < 2 * per_tensor; c += kThreads) {
    const int which = c >= per_tensor;
    const int cc = c - which * per_tensor;
    const int head = cc / CH, part = cc - head * CH;
    const uint8_t* src = (which ? v_new : k_new) +
                         (static_cast<size_t>(t) * num_kv_heads + head) * ROW_BYTES + part * 16;
    uint8_t* dst = (which ? v_pages : k_pages) +
                   ((static_cast<size_t>(blk) * num_kv_heads + head) * block_size + slot) * ROW_BYTES +
                   part * 16;
    *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
  }
}

int log2i(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

int hip_check(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pa::set_error(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return pa::clear_error();
}

int check_attn_scalars(const char* who, int32_t num_seqs, int32_t hq, int32_t hkv, int32_t d,
                       int32_t bs, int32_t dtype, int32_t num_tasks, int32_t num_combines,
                       int32_t num_partials, size_t ws_bytes, const void* ws, int32_t max_blocks) {
  if (num_seqs < 0 || num_tasks < 0 || num_combines < 0 || num_partials < 0 || max_blocks < 0)
    return pa::set_error(PA_ERR_SHAPE, "%s: negative size", who);
  if (hq < 1 || hkv < 1 || hq % hkv)
    return pa::set_error(PA_ERR_SHAPE, "%s: Hq %d is not a positive multiple of Hkv %d", who, hq, hkv);
  if (hq / hkv > pa::kMaxGroup)
    return pa::set_error(PA_ERR_SHAPE, "%s: Hq/Hkv = %d exceeds %d", who, hq / hkv, pa::kMaxGroup);
  if (!pa::head_dim_ok(d)) return pa::set_error(PA_ERR_SHAPE, "%s: head_dim %d not in {64, 128}", who, d);
  if (!pa::block_size_ok(bs))
    return pa::set_error(PA_ERR_BLOCK_SIZE, "%s: block_size %d is not a power of two in [16, 256]", who, bs);
  if (dtype != PA_BF16 && dtype != PA_FP32) return pa::set_error(PA_ERR_DTYPE, "%s: dtype %d", who, dtype);
  if (num_combines > 0) {
    if (!ws) return pa::set_error(PA_ERR_NULL, "%s: workspace is NULL", who);
    const size_t need = pa_workspace_bytes(num_partials, d);
    if (ws_bytes < need)
      return pa::set_error(PA_ERR_CAPACITY, "%s: workspace %zu bytes < %zu needed", who, ws_bytes, need);
  }
  return PA_OK;
}

AttnArgs make_args(const void* q, const void* kp, const void* vp, const int32_t* bt,
                   int32_t max_blocks, const int32_t* cu, const int32_t* ctx, int32_t hq,
                   int32_t hkv, int32_t d, int32_t bs, float scale, const pa_task* tasks,
                   int32_t num_tasks, int32_t num_partials, void* ws, void* out) {
  AttnArgs a;
  a.q = q;
  a.k_pages = kp;
  a.v_pages = vp;
  a.block_table = bt;
  a.cu_seqlens = cu;
  a.context_lens = ctx;
  a.tasks = tasks;
  a.ws_acc = static_cast<float*>(ws);
  size_t acc_bytes = (static_cast<size_t>(num_partials) * d * sizeof(float) + 255) & ~size_t(255);
  a.ws_ml = ws ? reinterpret_cast<float*>(static_cast<char*>(ws) + acc_bytes) : nullptr;
  a.out = out;
  a.max_blocks = max_blocks;
  a.num_q_heads = hq;
  a.num_kv_heads = hkv;
  a.block_size = bs;
  a.bs_shift = log2i(bs);
  a.num_tasks = num_tasks;
  a.scale_log2 = scale * kLog2e;
  return a;
}

template <typename T, int D>
void launch_combine(const pa_combine* comb, int32_t n, const int32_t* cu, const AttnArgs& a,
                    hipStream_t st) {
  if (n > 0)
    hipLaunchKernelGGL((combine_kernel<T, D>), dim3(n), dim3(kThreads), 0, st, comb, cu, a.ws_acc,
                       a.ws_ml, static_cast<T*>(a.out), a.num_q_heads);
}

}  // namespace

extern "C" int reshape_and_cache(const void* k_new, const void* v_new, void* k_pages,
                                 void* v_pages, const int32_t* block_table,
                                 int32_t max_blocks_per_seq, const int32_t* cu_seqlens_q,
                                 const int32_t* context_lens, int32_t num_seqs,
                                 int32_t num_tokens, int32_t num_blocks, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t dtype,
                                 void* stream) {
  if (num_tokens < 0 || num_seqs < 0 || num_blocks < 0 || max_blocks_per_seq < 0)
    return pa::set_error(PA_ERR_SHAPE, "reshape_and_cache: negative size");
  if (num_kv_heads < 1 || !pa::head_dim_ok(head_dim))
    return pa::set_error(PA_ERR_SHAPE, "reshape_and_cache: Hkv %d, head_dim %d", num_kv_heads, head_dim);
  if (!pa::block_size_ok(block_size))
    return pa::set_error(PA_ERR_BLOCK_SIZE, "reshape_and_cache: block_size %d", block_size);
  if (dtype != PA_BF16 && dtype != PA_FP32)
    return pa::set_error(PA_ERR_DTYPE, "reshape_and_cache: dtype %d", dtype);
  if (num_tokens == 0) return pa::clear_error();
  if (!k_new || !v_new || !k_pages || !v_pages || !block_table || !cu_seqlens_q || !context_lens)
    return pa::set_error(PA_ERR_NULL, "reshape_and_cache: NULL pointer");
  if (num_seqs < 1) return pa::set_error(PA_ERR_SHAPE, "reshape_and_cache: tokens without sequences");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int row_bytes = head_dim * (dtype == PA_BF16 ? 2 : 4);
  const int shift = log2i(block_size);
#define PA_RC_LAUNCH(RB)                                                                        \
  hipLaunchKernelGGL(reshape_and_cache_kernel<RB>, dim3(num_tokens), dim3(kThreads), 0, st,    \
                     static_cast<const uint8_t*>(k_new), static_cast<const uint8_t*>(v_new),    \
                     static_cast<uint8_t*>(k_pages), static_cast<uint8_t*>(v_pages), block_table, \
                     max_blocks_per_seq, cu_seqlens_q, context_lens, num_seqs, num_kv_heads,     \
                     block_size, shift)
  switch (row_bytes) {
    case 128: PA_RC_LAUNCH(128); break;
    case 256: PA_RC_LAUNCH(256); break;
    default: PA_RC_LAUNCH(512); break;
  }
#undef PA_RC_LAUNCH
  return hip_check("reshape_and_cache");
}

extern "C" int paged_attn_decode(const void* q, const void* k_pages, const void* v_pages,
                                 const int32_t* block_table, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, float scale, int32_t dtype,
                                 const pa_task* tasks_dev, int32_t num_tasks,
                                 const pa_combine* combines_dev, int32_t num_combines,
                                 int32_t num_partials, void* workspace, size_t workspace_bytes,
                                 void* out, void* stream) {
  if (int rc = check_attn_scalars("paged_attn_decode", num_seqs, num_q_heads, num_kv_heads,
                                  head_dim, block_size, dtype, num_tasks, num_combines,
                                  num_partials, workspace_bytes, workspace, max_blocks_per_seq))
    return rc;
  if (num_tasks == 0) return pa::clear_error();
  if (!q || !k_pages || !v_pages || !block_table || !out || !tasks_dev ||
      (num_combines > 0 && !combines_dev))
    return pa::set_error(PA_ERR_NULL, "paged_attn_decode: NULL pointer");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const AttnArgs a = make_args(q, k_pages, v_pages, block_table, max_blocks_per_seq, nullptr,
                               context_lens, num_q_heads, num_kv_heads, head_dim, block_size,
                               scale, tasks_dev, num_tasks, num_partials, workspace, out);
  if (dtype == PA_BF16) {
    if (head_dim == 128) {
      hipLaunchKernelGGL((decode_kernel<__bf16, 128>), dim3(num_tasks), dim3(kThreads), 0, st, a);
      launch_combine<__bf16, 128>(combines_dev, num_combines, nullptr, a, st);
    } else {
      hipLaunchKernelGGL((decode_kernel<__bf16, 64>), dim3(num_tasks), dim3(kThreads), 0, st, a);
      launch_combine<__bf16, 64>(combines_dev, num_combines, nullptr, a, st);
    }
  } else {
    if (head_dim == 128) {
      hipLaunchKernelGGL((decode_kernel<float, 128>), dim3(num_tasks), dim3(kThreads), 0, st, a);
      launch_combine<float, 128>(combines_dev, num_combines, nullptr, a, st);
    } else {
      hipLaunchKernelGGL((decode_kernel<float, 64>), dim3(num_tasks), dim3(kThreads), 0, st, a);
      launch_combine<float, 64>(combines_dev, num_combines, nullptr, a, st);
    }
  }
  return hip_check("paged_attn_decode");
}

extern "C" int paged_attn_varlen_prefill(
    const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
    int32_t max_blocks_per_seq, const int32_t* cu_seqlens_q, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, float scale, int32_t dtype, const pa_task* tasks_dev,
    int32_t num_tasks, const pa_combine* combines_dev, int32_t num_combines,
    int32_t num_partials, void* workspace, size_t workspace_bytes, void* out, void* stream) {
  if (int rc = check_attn_scalars("paged_attn_varlen_prefill", num_seqs, num_q_heads,
                                  num_kv_heads, head_dim, block_size, dtype, num_tasks,
                                  num_combines, num_partials, workspace_bytes, workspace,
                                  max_blocks_per_seq))
    return rc;
  if (dtype != PA_BF16)
    return pa::set_error(PA_ERR_DTYPE, "paged_attn_varlen_prefill: the MFMA path needs PA_BF16");
  if (num_tokens < num_seqs)
    return pa::set_error(PA_ERR_SHAPE, "paged_attn_varlen_prefill: %d tokens for %d sequences",
                         num_tokens, num_seqs);
  if (num_tasks == 0) return pa::clear_error();
  if (!q || !k_pages || !v_pages || !block_table || !cu_seqlens_q || !context_lens || !out ||
      !tasks_dev || (num_combines > 0 && !combines_dev))
    return pa::set_error(PA_ERR_NULL, "paged_attn_varlen_prefill: NULL pointer");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const AttnArgs a = make_args(q, k_pages, v_pages, block_table, max_blocks_per_seq,
                               cu_seqlens_q, context_lens, num_q_heads, num_kv_heads, head_dim,
                               block_size, scale, tasks_dev, num_tasks, num_partials, workspace,
                               out);
  if (head_dim == 128) {
    hipLaunchKernelGGL(meta_attn_kernel<128>, dim3(num_tasks), dim3(kThreads), 0, st, a);
    launch_combine<__bf16, 128>(combines_dev, num_combines, cu_seqlens_q, a, st);
  } else {
    hipLaunchKernelGGL(meta_attn_kernel<64>, dim3(num_tasks), dim3(kThreads), 0, st, a);
    launch_combine<__bf16, 64>(combines_dev, num_combines, cu_seqlens_q, a, st);
  }
  return hip_check("paged_attn_varlen_prefill");
}
