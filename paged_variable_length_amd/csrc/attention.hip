// HIP kernels and launchers of libpagedattn.so, written for gfx950 (MI355X, CDNA4).
//
// Kernels
//   reshape_and_cache_kernel      copy of new K/V rows into their page slots (HBM-bound copy)
//   reshape_and_cache_fp8_kernel  the same into fp8 pages: each touched page is re-encoded
//                                 with a power-of-two scale covering its old and new rows
//   decode_kernel                 split-K decode attention, one workgroup per decode task
//   decode_fp8_kernel             the same over fp8 pages (codes converted in registers)
//   meta_attn_kernel              one grid over a mixed, load-sorted task table: each
//                                 workgroup reads its task's kind and runs the decode or the
//                                 prefill body
//   meta_attn_fp8_kernel          the same over fp8 pages
//   combine_kernel                log-sum-exp merge of split partials into `out`
//
// Decode body (HBM-bound). A task is (sequence, kv head, key range). Its four waves take
// interleaved chunks of the key range. Scores S = K Q^T come from 16x16x32 bf16 MFMAs whose
// 16 columns are the G query heads of the kv head (zero-padded to 16), so every K/V page is
// read once for all heads of its group. K rows are loaded straight into the MFMA operand
// layout; V rows are loaded 16 bytes per lane along D and rearranged in registers, so the
// value product O^T = V^T P^T consumes them without an LDS round trip and each lane ends up
// owning one head's slice of D. Online softmax in base 2, per head; the four waves merge
// through LDS at the end and write either the output row or an fp32 partial. Block ids come
// from scalar loads a chunk ahead; page reads carry the non-temporal hint where nothing in the
// launch re-reads them (decode tables, and unified tables without prefill tiles), and a wave
// keeps one chunk of reads in flight (three waves per SIMD, tables with shared-prefix tasks)
// or two (two waves per SIMD, everything else).
//
// Prefill body (MFMA-bound). A task is (sequence, query head, up to 128 query rows, key
// range). 64-key K and V tiles are gathered through the block table into two LDS buffers
// each; each wave owns 32 query rows, computes S^T = K Q^T and O^T += V^T P^T with 32x32x16
// bf16 MFMAs, and applies the causal mask only on tiles that cross the diagonal. The tile
// loop is software-pipelined: the scores of tile j+1 are formed while the exponentials of
// tile j are, and the value product of tile j runs beside the maximum of tile j+1. Each
// iteration's direct loads are issued together right after its barrier. Over fp8 pages the
// tiles hold the codes themselves at D = 128 (converted with the page scales at the operand
// reads) and converted bf16 values at D = 64 (converted on their way into LDS).
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
// read-only data reached through the constant address space, so uniform indexes load it
// with scalar loads
typedef __attribute__((address_space(4))) const int32_t cint32;
typedef __attribute__((address_space(4))) const float cfloat;

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
  const float* scales;          // fp8 pages: [num_blocks, Hkv, 2] (K, V) scales per page
  int32_t max_blocks;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t bs_shift;
  int32_t num_tasks;
  float scale_log2;             // softmax scale * log2(e)
  int32_t stream_reads;         // unified launch: decode page reads non-temporal (no prefill tiles)
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Two E4M3FN codes (bytes 0,1 of w, or 2,3 with hi) times a page scale 2^k, as two bf16
// values. The conversion applies the exponent of its scale operand; for a power of two that
// is the exact product, and every E4M3FN value times 2^k (k >= -120) is a bf16 value (a
// subnormal one at the bottom of the range), so nothing rounds.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, HI));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Low (k even) or high (k odd) bf16 halves of two dwords, packed as (a_half, b_half).
__device__ __forceinline__ uint32_t pair_half(uint32_t a, uint32_t b, int odd) {
  return odd ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
}

// ------------------------------------------------------------------------------------------
// Decode body, bf16; also runs verify tasks (all R <= 16/G rows of a short sequence).
// Score column i16 is (row i16 / G, head i16 % G) of the task's R*G columns; for decode R = 1
// and the columns are the G query heads. Lane map inside a wave: i16 = lane & 15, g4 = lane >> 4.
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

// Float index of (row, d) in the merge buffer sm_acc ([4 waves x 16 columns] rows of D). Each
// lane stores its column's d = VEC*(4*g4 + r) + n for fixed (r, n) in one instruction, so
// unpadded rows (D floats, a multiple of the bank count) would put the 16 columns of a lane
// group in one bank. Rows of D + 1 floats spread them: at D = 64 the 64 lanes of a store hit
// 64 distinct banks; at D = 128, lanes g4 and g4 + 2 of one column (64 floats apart) still share
// a bank, a two-way conflict where there were sixteen. The merge's reads (consecutive d of one
// row) stay contiguous.
template <int D>
__device__ __forceinline__ int merge_idx(int row, int d) {
  return row * (D + 1) + d;
}
// floats of the decode merge buffers: sm_m, sm_l [4][16] each, sm_acc [64 padded rows]
template <int D>
constexpr int kMergeFloats = 128 + 64 * (D + 1);

// Merge of the four waves' partial states per score column, then the output row or an fp32
// partial. Column c is (row c / G, head c % G); rows are relative to packed row tok.
template <int D>
__device__ __forceinline__ void decode_merge_and_store(const AttnArgs& a, const pa_task& t,
                                                       int tok, int G, int ncol, float m,
                                                       float l, const f32x4* acc, float* smem,
                                                       bool out_bf16) {
  constexpr int VEC = D / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g4 = lane >> 4;
  l += wave_shfl_xor(l, 16);
  l += wave_shfl_xor(l, 32);
  float* sm_m = smem;              // [4][16]
  float* sm_l = smem + 64;         // [4][16]
  float* sm_acc = smem + 128;      // [4][16] padded rows of D (merge_idx)
  if (g4 == 0) {
    sm_m[wave * 16 + i16] = m;
    sm_l[wave * 16 + i16] = l;
  }
  if (i16 < ncol) {
#pragma unroll
    for (int n = 0; n < VEC; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sm_acc[merge_idx<D>(wave * 16 + i16, VEC * (4 * g4 + r) + n)] = acc[n][r];
  }
  __syncthreads();
  const int hq0 = t.head * G;
  for (int idx = threadIdx.x; idx < ncol * D; idx += kThreads) {
    const int h = idx / D, d = idx - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w * 16 + h]);
    // a verify row may see no key of this split in any wave: weight 0 (m = -inf, l = 0)
    const float Muse = M == -INFINITY ? 0.f : M;
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float wt = fast_exp2(sm_m[w * 16 + h] - Muse);
      L += wt * sm_l[w * 16 + h];
      A += wt * sm_acc[merge_idx<D>(w * 16 + h, d)];
    }
    if (t.partial < 0) {
      const int row = h / G, hh = h - row * G;
      const size_t o = (static_cast<size_t>(tok + row) * a.num_q_heads + hq0 + hh) * D + d;
      const float v = A / L;
      if (out_bf16)
        static_cast<__bf16*>(a.out)[o] = static_cast<__bf16>(v);
      else
        static_cast<float*>(a.out)[o] = v;
    } else {
      // shared-prefix tasks: member h / G's rows start q_row0 (the member stride) apart
      const int mem = h / G;
      const size_t row = static_cast<size_t>(t.partial) +
                         (t.kind == PA_TASK_SHARED ? mem * t.q_row0 + (h - mem * G) : h);
      a.ws_acc[row * D + d] = A;
      if (d == 0) {
        a.ws_ml[2 * row] = M;
        a.ws_ml[2 * row + 1] = L;
      }
    }
  }
}

// A page read; NT marks it non-temporal (the line is a first candidate for eviction), for page
// streams that are read once per launch and should not push reused lines out of the caches.
template <bool NT, typename T>
__device__ __forceinline__ T ld(const T* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

template <int D, bool AHEAD, bool NT>
__device__ void decode_task_bf16(const AttnArgs& a, const pa_task& t, float* smem) {
  constexpr int KS = D / 32;
  constexpr int VEC = D / 16;
  typedef typename DecodeVRaw<D>::type VRaw;
  const int lane = threadIdx.x & 63;
  // wave-uniform: chunk indices, tile bounds and block ids stay in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i16 = lane & 15, g4 = lane >> 4;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int s = t.seq, kvh = t.head;
  const int tok = a.cu_seqlens ? a.cu_seqlens[s] : s;
  const int bs = a.block_size;
  // rows: 1 for decode, the draft rows for verify, the members (consecutive decode rows, so
  // member r's row is tok + r) for a shared-prefix task
  const int nrows = t.q_rows;
  const int ncol = nrows * G;
  const int row = i16 / G, hh = i16 - row * G;     // this lane's score column

  bf16x8 qf[KS];
  {
    const uint16_t* qp =
        static_cast<const uint16_t*>(a.q) +
        (static_cast<size_t>(tok + row) * a.num_q_heads + kvh * G + hh) * D + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (i16 < ncol) v = *reinterpret_cast<const u32x4*>(qp + 32 * ks);
      qf[ks] = as_bf16x8(v);
    }
  }
  // causal limit of this column: its row sits at position ctx - nrows + row and sees the keys
  // before that position and the key at it (for decode: every key). A shared-prefix task's
  // rows are single decode rows of its members, and its keys lie below every member's own
  // row: no limit.
  const bool shared = t.kind == PA_TASK_SHARED;
  const int key_lim = shared ? INT_MAX : a.context_lens[s] - nrows + row + 1;
  const int lim_lo = shared ? INT_MAX : a.context_lens[s] - nrows + 1;
  const size_t head_stride = static_cast<size_t>(bs) * D;
  const size_t block_stride = static_cast<size_t>(a.num_kv_heads) * head_stride;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k_pages) + kvh * head_stride;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v_pages) + kvh * head_stride;
  cint32* bt = (cint32*)(a.block_table + static_cast<size_t>(s) * a.max_blocks);
  const float c = a.scale_log2;

  f32x4 acc[VEC];
#pragma unroll
  for (int n = 0; n < VEC; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  const int kv0 = t.kv0, kv1 = t.kv1;
  const int nchunks = (kv1 - kv0 + 31) >> 5;
  // block ids of a chunk's two 16-key tiles, by scalar loads one chunk ahead of their use. A
  // tile past kv1 takes the block of key kv1 - 1: its loads read rows of a valid page, and the
  // tail masking below gives them no weight.
  auto chunk_blocks = [&](int ch, int (&blk)[2]) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) blk[tt] = bt[min(kv0 + 32 * ch + 16 * tt, kv1 - 1) >> a.bs_shift];
  };
  auto load_chunk = [&](int ch, const int (&blk)[2], bf16x8 (&kf)[2][KS], VRaw (&vr)[8]) {
    const int cs = kv0 + 32 * ch;
    size_t off[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
      off[tt] = static_cast<size_t>(blk[tt]) * block_stride +
                static_cast<size_t>((cs + 16 * tt) & (bs - 1)) * D;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kf[tt][ks] = as_bf16x8(ld<NT>(
            reinterpret_cast<const u32x4*>(kbase + off[tt] + i16 * D + 32 * ks + 8 * g4)));
#pragma unroll
    for (int e = 0; e < 8; ++e)
      vr[e] = ld<NT>(reinterpret_cast<const VRaw*>(
          vbase + off[e >> 2] + (4 * g4 + (e & 3)) * D + VEC * i16));
  };
  auto compute_chunk = [&](int ch, const bf16x8 (&kf)[2][KS], VRaw (&vr)[8]) {
    const int cs = kv0 + 32 * ch;
    f32x4 sc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      sc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        sc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[tt][ks], qf[ks], sc[tt], 0, 0, 0);
    }
    if (cs + 32 > kv1) {
      // tail chunk: keys past kv1 get no weight, and the values loaded for them (rows of some
      // valid page, possibly non-finite) are replaced by zeros so that 0 * value stays 0 in the
      // value product
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = cs + 16 * (e >> 2) + 4 * g4 + (e & 3);
        if (key >= kv1) {
          sc[e >> 2][e & 3] = -INFINITY;
          vr[e] = VRaw{};
        }
      }
    }
    if (cs + 32 > lim_lo) {
      // keys after a verify row's own position get no weight in that row's column (their
      // values are finite: they lie below kv1)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = cs + 16 * (e >> 2) + 4 * g4 + (e & 3);
        if (key >= key_lim) sc[e >> 2][e & 3] = -INFINITY;
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
  };
  // A wave takes chunks wave, wave + 4, ...; with AHEAD it issues the loads of its next chunk
  // before it computes the current one (two register sets, taken in turn), so two chunks of
  // loads are in flight per wave.
  int blk[2];
  chunk_blocks(wave, blk);
  if constexpr (AHEAD) {
    bf16x8 ka[2][KS], kb[2][KS];
    VRaw va[8], vb[8];
    if (wave < nchunks) load_chunk(wave, blk, ka, va);
    chunk_blocks(wave + 4, blk);
    for (int ch = wave; ch < nchunks; ch += 8) {
      if (ch + 4 < nchunks) load_chunk(ch + 4, blk, kb, vb);
      chunk_blocks(ch + 8, blk);
      compute_chunk(ch, ka, va);
      if (ch + 4 >= nchunks) break;
      if (ch + 8 < nchunks) load_chunk(ch + 8, blk, ka, va);
      chunk_blocks(ch + 12, blk);
      compute_chunk(ch + 4, kb, vb);
    }
  } else {
    for (int ch = wave; ch < nchunks; ch += 4) {
      bf16x8 kf[2][KS];
      VRaw vr[8];
      load_chunk(ch, blk, kf, vr);
      chunk_blocks(ch + 4, blk);
      compute_chunk(ch, kf, vr);
    }
  }
  decode_merge_and_store<D>(a, t, tok, G, ncol, m, l, acc, smem, true);
}

// ------------------------------------------------------------------------------------------
// Decode body over fp8 pages: OCP E4M3FN codes with one power-of-two scale per (block, kv head)
// page for K and one for V. Lane maps, softmax and outputs follow the bf16 body, except:
//   QK: lane (i16, g4) loads 16 codes of key i16 at d = 64*j + 16*g4 (j < D/64); codes 0..7
//       are its operand of k-step 2j, codes 8..15 of k-step 2j+1, and q is read in the same d
//       order, so each dot product is the same sum;
//   every code becomes bf16 with its page scale applied in the same exact conversion;
//   a wave loads the raw codes of its next chunk before it computes the current one, and the
//   block ids of the chunk after that, so a chunk of loads is always in flight per wave.
// Decode, verify and shared-prefix tasks: as in the bf16 body, the 16 columns are (query row,
// head) pairs of the task's q_rows rows (one for decode; the members' single rows for a shared
// prefix), each masking the keys after its row's position (a shared prefix lies below every
// member's row: no limit).
// ------------------------------------------------------------------------------------------
template <int D>
struct Fp8VRaw;
template <>
struct Fp8VRaw<128> {
  typedef u32x2 type;  // 8 codes along D
};
template <>
struct Fp8VRaw<64> {
  typedef uint32_t type;  // 4 codes along D
};

template <int D>
struct Fp8Chunk {
  u32x4 k[2][D / 64];               // [tile][j]: 16 codes of key i16 at d = 64*j + 16*g4
  typename Fp8VRaw<D>::type v[8];   // slot e: key (tile e>>2, row 4*g4 + (e&3)), d = VEC*i16 + ..
  float ksc[2], vsc[2];             // page scales of the two tiles
};

// dword w of a V slot (w < D/64): the whole slot for D = 64
template <int D>
__device__ __forceinline__ uint32_t vslot_word(const typename Fp8VRaw<D>::type& v, int w) {
  if constexpr (D == 128)
    return v[w];
  else
    return v;
}

template <int D, bool NT>
__device__ void decode_task_fp8(const AttnArgs& a, const pa_task& t, float* smem) {
  constexpr int KS = D / 32;
  constexpr int KJ = D / 64;
  constexpr int VEC = D / 16;
  typedef typename Fp8VRaw<D>::type VRaw;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i16 = lane & 15, g4 = lane >> 4;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int s = t.seq, kvh = t.head;
  const int tok = a.cu_seqlens ? a.cu_seqlens[s] : s;
  const int bs = a.block_size;
  const int nrows = t.q_rows;
  const int ncol = nrows * G;
  const int row = i16 / G, hh = i16 - row * G;     // this lane's score column

  bf16x8 qf[KS];
  {
    const uint16_t* qp =
        static_cast<const uint16_t*>(a.q) +
        (static_cast<size_t>(tok + row) * a.num_q_heads + kvh * G + hh) * D + 16 * g4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (i16 < ncol) v = *reinterpret_cast<const u32x4*>(qp + 64 * (ks >> 1) + 8 * (ks & 1));
      qf[ks] = as_bf16x8(v);
    }
  }
  // causal limit of this column (its row sits at position ctx - nrows + row; decode: every key)
  const bool shared = t.kind == PA_TASK_SHARED;
  const int key_lim = shared ? INT_MAX : a.context_lens[s] - nrows + row + 1;
  const int lim_lo = shared ? INT_MAX : a.context_lens[s] - nrows + 1;
  const size_t head_stride = static_cast<size_t>(bs) * D;
  const size_t block_stride = static_cast<size_t>(a.num_kv_heads) * head_stride;
  const uint8_t* kbase = static_cast<const uint8_t*>(a.k_pages) + kvh * head_stride;
  const uint8_t* vbase = static_cast<const uint8_t*>(a.v_pages) + kvh * head_stride;
  const int32_t* bt = a.block_table + static_cast<size_t>(s) * a.max_blocks;
  const float c = a.scale_log2;
  const int kv0 = t.kv0, kv1 = t.kv1;
  const int nchunks = (kv1 - kv0 + 31) >> 5;

  // block ids of chunk ch's two tiles; a tile at or past kv1 takes the block of key kv1 - 1,
  // so its (weightless) loads stay inside the sequence's own pages
  auto ids = [&](int ch, int (&blk)[2]) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) blk[tt] = bt[min(kv0 + 32 * ch + 16 * tt, kv1 - 1) >> a.bs_shift];
  };
  auto load = [&](int ch, const int (&blk)[2], Fp8Chunk<D>& r) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int ts = kv0 + 32 * ch + 16 * tt;
      const size_t off =
          static_cast<size_t>(blk[tt]) * block_stride + static_cast<size_t>(ts & (bs - 1)) * D;
#pragma unroll
      for (int j = 0; j < KJ; ++j)
        r.k[tt][j] = ld<NT>(reinterpret_cast<const u32x4*>(kbase + off + i16 * D + 64 * j + 16 * g4));
#pragma unroll
      for (int e = 0; e < 4; ++e)
        r.v[4 * tt + e] =
            ld<NT>(reinterpret_cast<const VRaw*>(vbase + off + (4 * g4 + e) * D + VEC * i16));
      // the K and V scales of a page sit side by side: one 8-byte read
      const size_t page = static_cast<size_t>(blk[tt]) * a.num_kv_heads + kvh;
      const f32x2 sc = *reinterpret_cast<const f32x2*>(a.scales + 2 * page);
      r.ksc[tt] = sc[0];
      r.vsc[tt] = sc[1];
    }
  };

  f32x4 acc[VEC];
#pragma unroll
  for (int n = 0; n < VEC; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  auto compute = [&](int ch, const Fp8Chunk<D>& r) {
    const int cs = kv0 + 32 * ch;
    f32x4 sc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      sc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KJ; ++j) {
        const u32x4 w = r.k[tt][j];
        const float ks = r.ksc[tt];
        const u32x4 lo = {fp8x2_to_bf16x2<false>(w[0], ks), fp8x2_to_bf16x2<true>(w[0], ks),
                          fp8x2_to_bf16x2<false>(w[1], ks), fp8x2_to_bf16x2<true>(w[1], ks)};
        const u32x4 hi = {fp8x2_to_bf16x2<false>(w[2], ks), fp8x2_to_bf16x2<true>(w[2], ks),
                          fp8x2_to_bf16x2<false>(w[3], ks), fp8x2_to_bf16x2<true>(w[3], ks)};
        sc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(lo), qf[2 * j], sc[tt], 0, 0, 0);
        sc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(hi), qf[2 * j + 1], sc[tt], 0, 0, 0);
      }
    }
    VRaw vr[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) vr[e] = r.v[e];
    if (cs + 32 > kv1) {
      // tail chunk: keys past kv1 get no weight, and their codes become +0 so that
      // 0 * value stays 0 in the value product
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = cs + 16 * (e >> 2) + 4 * g4 + (e & 3);
        if (key >= kv1) {
          sc[e >> 2][e & 3] = -INFINITY;
          vr[e] = VRaw{};
        }
      }
    }
    if (cs + 32 > lim_lo) {
      // keys after a verify row's own position get no weight in that row's column (their
      // values are finite: they lie below kv1)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = cs + 16 * (e >> 2) + 4 * g4 + (e & 3);
        if (key >= key_lim) sc[e >> 2][e & 3] = -INFINITY;
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mx = fmaxf(mx, wave_shfl_xor(mx, 16));
    mx = fmaxf(mx, wave_shfl_xor(mx, 32));
    const float mnew = fmaxf(m, mx * c);
    // a verify column can have seen no key yet (every score -inf): weights 0, not NaN
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
    const u32x4 pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                      pack_bf16x2(p[6], p[7])};
    const bf16x8 pf = as_bf16x8(pw);
    // byte-interleaved slot pairs: pr[qd][w][h] holds value n = 4*w + 2*h + (0, 1) of slots
    // 2*qd and 2*qd + 1 as bytes (slot 2qd, slot 2qd+1, slot 2qd, slot 2qd+1)
    uint32_t pr[4][KJ][2];
#pragma unroll
    for (int qd = 0; qd < 4; ++qd)
#pragma unroll
      for (int w = 0; w < KJ; ++w) {
        const uint32_t ev = vslot_word<D>(vr[2 * qd], w), od = vslot_word<D>(vr[2 * qd + 1], w);
        pr[qd][w][0] = __builtin_amdgcn_perm(od, ev, 0x05010400u);
        pr[qd][w][1] = __builtin_amdgcn_perm(od, ev, 0x07030602u);
      }
#pragma unroll
    for (int n = 0; n < VEC; ++n) {
      u32x4 vw;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        vw[qd] = (n & 1) ? fp8x2_to_bf16x2<true>(pr[qd][n >> 2][(n >> 1) & 1], r.vsc[qd >> 1])
                         : fp8x2_to_bf16x2<false>(pr[qd][n >> 2][(n >> 1) & 1], r.vsc[qd >> 1]);
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vw), pf, acc[n], 0, 0, 0);
    }
  };

  if (wave < nchunks) {
    // two register buffers in turn (no copies, which would wait for the loads in flight)
    int ch = wave;
    int bn[2], bn2[2];
    Fp8Chunk<D> ca, cb;
    ids(ch, bn);
    load(ch, bn, ca);
    ids(ch + 4, bn);
    while (true) {
      if (ch + 4 >= nchunks) {
        compute(ch, ca);
        break;
      }
      ids(ch + 8, bn2);
      load(ch + 4, bn, cb);
      compute(ch, ca);
      ch += 4;
      bn[0] = bn2[0];
      bn[1] = bn2[1];
      if (ch + 4 >= nchunks) {
        compute(ch, cb);
        break;
      }
      ids(ch + 8, bn2);
      load(ch + 4, bn, ca);
      compute(ch, cb);
      ch += 4;
      bn[0] = bn2[0];
      bn[1] = bn2[1];
    }
  }
  decode_merge_and_store<D>(a, t, tok, G, ncol, m, l, acc, smem, true);
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
  // columns: the G heads of one decode row, or (member, head) pairs of a shared-prefix task
  // (members are consecutive decode rows, so member r's row is tok + r)
  const int ncol = t.q_rows * G;
  const int row = i16 / G, hh = i16 - row * G;

  f32x4 qf[KQ];
  {
    const float* qp = static_cast<const float*>(a.q) +
                      (static_cast<size_t>(tok + row) * a.num_q_heads + kvh * G + hh) * D + 4 * g4;
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq) {
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (i16 < ncol) v = *reinterpret_cast<const f32x4*>(qp + 16 * kq);
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
  decode_merge_and_store<D>(a, t, tok, G, ncol, m, l, acc, smem, false);
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
// instruction) into [K buffer 0 | K buffer 1 | V buffer 0 | V buffer 1]; K runs two tiles
// ahead of its use and V one. Rows are stored unpadded with the 16-byte chunks of key row k
// permuted by XOR with lds_swz(k), so the K reads and the transposed V reads spread over the
// banks.
// V^T operands come from ds_read_b64_tr_b16: within each 16-lane group, lane j = 4r + c
// returns element c of the 8-byte segments addressed by lanes r, 4+r, 8+r, 12+r. With lane k
// of the group addressing key kbase + k/4, d = d0 + 4*(k%4), lane j receives the four keys
// kbase .. kbase+3 at d = d0 + j -- a column of V, as the MFMA operand needs.
// Lane-dependent LDS addresses are computed once per task; buffer, key block and k-step
// enter as instruction offsets or as one XOR on a single base register.
// ------------------------------------------------------------------------------------------
// CODES: the tiles hold fp8 codes (1 byte per element) instead of bf16 values.
template <int D, bool CODES = false>
struct PrefillCfg {
  static constexpr int kTile = 64;                                  // keys per LDS tile
  static constexpr int kRowBytes = CODES ? D : D * 2;               // one key row
  static constexpr int kChunks = kRowBytes / 16;                    // 16-byte chunks per row
  static constexpr int kTileBytes = kTile * kRowBytes;
  static constexpr int kKeysPerLoad = 1024 / kRowBytes;             // keys per wave load
  static constexpr int kLoadsPerWave = kTileBytes / 1024 / 4;       // per tensor per tile
  static constexpr size_t kSmemBytes = 4 * static_cast<size_t>(kTileBytes);  // 2 K + 2 V
};

// XOR pattern of the 16-byte chunks of key row `key` (a permutation of the row's chunks).
// With 16 chunks per row (D = 128), chunk bits 2-3 follow key bits 0-1 and chunk bits 0-1
// follow key bits 2-3: sixteen consecutive keys reading one chunk hit sixteen distinct
// chunk positions, and the transposed reads (four keys x four neighbouring chunks) hit
// sixteen distinct positions too. Measured on gfx950 with eight waves per CU, this halves the
// LDS time of both read patterns against a 3-bit pattern and matches an unswizzled
// contiguous read. With 8 chunks per row (D = 64) a 3-bit pattern is used. The pattern
// depends on key & 15 only, so shifting a key by a multiple of 16 keeps its pattern.
// Rows of fp8 codes (CODES, D = 128: 8 chunks of 16 codes): chunk c of key row r sits at
// c ^ s(r), s(r) = 2*r1 + r2 + 4*r3 for key bits r1, r2, r3. With 64 banks of 4 bytes a row
// covers half the banks, so rows of opposite parity share a bank line. Sixteen consecutive rows
// reading one chunk (the K operand reads) take the eight chunk positions within each parity
// (s is a permutation of 0..7 over bits 1-3); a transposed read takes rows {4g + 0..3,
// 8 + 4g + 0..3} (g = 0, 1) at two neighbouring chunks, and s >> 1 differs between the four
// rows of each parity there, so its sixteen half-chunk segments per parity meet no bank twice.
template <int D, bool CODES = false>
__device__ __forceinline__ int lds_swz(int key) {
  if constexpr (CODES)
    return 2 * ((key >> 1) & 1) + ((key >> 2) & 1) + 4 * ((key >> 3) & 1);
  else if constexpr (D == 128)
    return ((key & 3) << 2) | ((key >> 2) & 3);
  else
    return ((key & 3) << 1) | ((key >> 2) & 1);
}

// Batches of N (4 or 8) LDS reads of one kind at lane addresses a[i] plus the byte offset
// OFF, written as asm: the compiler cannot tell that these reads never touch the buffer the
// direct loads are filling and would otherwise wait for those loads before each read.
// `_issue` only issues the reads. `lds_wait<K>` then waits until at most K LDS operations are
// outstanding and ties the batch's registers, so nothing reads them before the data arrived.
// LDS operations complete in issue order, so with K = the number of reads issued after a
// batch, that batch is complete; other counted operations in between only make the wait
// stronger. The compiler's own waits stay valid: extra outstanding operations are older.
#define PA_LDS_READ(OP, T)                                                                    \
  template <int OFF>                                                                          \
  __device__ __forceinline__ void OP##_x8_issue(const uint32_t (&a)[8], T (&r)[8]) {          \
    asm volatile(#OP " %0, %8 offset:%16\n\t" #OP " %1, %9 offset:%16\n\t"                   \
                 #OP " %2, %10 offset:%16\n\t" #OP " %3, %11 offset:%16\n\t"                  \
                 #OP " %4, %12 offset:%16\n\t" #OP " %5, %13 offset:%16\n\t"                  \
                 #OP " %6, %14 offset:%16\n\t" #OP " %7, %15 offset:%16"                      \
                 : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]),           \
                   "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])                                      \
                 : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]),          \
                   "v"(a[6]), "v"(a[7]), "n"(OFF)                                             \
                 : "memory");                                                                 \
  }                                                                                           \
  template <int OFF>                                                                          \
  __device__ __forceinline__ void OP##_x4_issue(const uint32_t (&a)[4], T (&r)[4]) {          \
    asm volatile(#OP " %0, %4 offset:%8\n\t" #OP " %1, %5 offset:%8\n\t"                     \
                 #OP " %2, %6 offset:%8\n\t" #OP " %3, %7 offset:%8"                          \
                 : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])                         \
                 : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "n"(OFF)                       \
                 : "memory");                                                                 \
  }
PA_LDS_READ(ds_read_b128, u32x4)
PA_LDS_READ(ds_read_b64_tr_b16, u32x2)
// ds_read_b64_tr_b8 (probed on gfx950): within each 16-lane group, lane j = 8r + c returns
// byte c of the 8-byte segments addressed by lanes r, r+2, ..., r+14. With lane k of the group
// addressing key kbase + k/2, byte offset d0 + 8*(k%2) of a row of codes, lane j receives the
// eight keys kbase .. kbase+7 at d = d0 + j.
PA_LDS_READ(ds_read_b64_tr_b8, u32x2)
#undef PA_LDS_READ

template <int K, typename T>
__device__ __forceinline__ void lds_wait(T (&r)[8]) {
  asm volatile("s_waitcnt lgkmcnt(%8)"
               : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]),
                 "+v"(r[6]), "+v"(r[7])
               : "n"(K)
               : "memory");
}
template <int K, typename T>
__device__ __forceinline__ void lds_wait(T (&r)[4]) {
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3])
               : "n"(K)
               : "memory");
}

// Causal mask of one 32-key block of S^T scores: register r holds key offset
// BASE + 8*(r/4) + r%4 (plus the lane's own offset, folded into lim); offsets >= lim become
// -inf. Written as compare/select pairs on VCC so no lane masks pile up in scalar registers.
template <int OFF>
__device__ __forceinline__ float mask_one(float x, int lim, float ninf) {
  asm("v_cmp_lt_i32_e32 vcc, %2, %1\n\tv_cndmask_b32_e32 %0, %3, %0, vcc"
      : "+v"(x)
      : "v"(lim), "n"(OFF), "v"(ninf)
      : "vcc");
  return x;
}
template <int BASE>
__device__ __forceinline__ void mask_block(f32x16& s, int lim) {
  const float ninf = -INFINITY;
  s[0] = mask_one<BASE + 0>(s[0], lim, ninf);    s[1] = mask_one<BASE + 1>(s[1], lim, ninf);
  s[2] = mask_one<BASE + 2>(s[2], lim, ninf);    s[3] = mask_one<BASE + 3>(s[3], lim, ninf);
  s[4] = mask_one<BASE + 8>(s[4], lim, ninf);    s[5] = mask_one<BASE + 9>(s[5], lim, ninf);
  s[6] = mask_one<BASE + 10>(s[6], lim, ninf);   s[7] = mask_one<BASE + 11>(s[7], lim, ninf);
  s[8] = mask_one<BASE + 16>(s[8], lim, ninf);   s[9] = mask_one<BASE + 17>(s[9], lim, ninf);
  s[10] = mask_one<BASE + 18>(s[10], lim, ninf); s[11] = mask_one<BASE + 19>(s[11], lim, ninf);
  s[12] = mask_one<BASE + 24>(s[12], lim, ninf); s[13] = mask_one<BASE + 25>(s[13], lim, ninf);
  s[14] = mask_one<BASE + 26>(s[14], lim, ninf); s[15] = mask_one<BASE + 27>(s[15], lim, ninf);
}

// MODE 0: bf16 pages. MODE 1 (FP8) and 2 (CODES): the pages hold E4M3FN codes with a
// power-of-two scale per page and tensor.
// FP8: a wave loads its share of a tile into registers (8 codes per lane and piece, the same
// elements the direct load would move), and after the tile's compute converts them exactly to
// bf16 and writes them where the direct load would have put them: the LDS layout, the buffers
// and the compute are those of the bf16 pages.
// CODES (D = 128): the direct loads move the codes themselves into LDS (half the bytes of a
// bf16 tile) and every operand read converts them: a K read returns 16 codes of one key (the
// operands of two k-steps, in a permuted d order that q follows), a transposed V read 8 keys
// of one d; each is converted with the scale of its key's page. The loads, buffers and their
// protocol are those of the bf16 pages.
template <int D, int MODE = 0>
__device__ void prefill_task(const AttnArgs& a, const pa_task& t, char* smem) {
  constexpr bool FP8 = MODE == 1;
  constexpr bool CODES = MODE == 2;
  static_assert(!CODES || D == 128, "codes in LDS are laid out for D = 128");
  typedef PrefillCfg<D, CODES> C;
  constexpr int KS = D / 16;   // k-steps of the QK product
  constexpr int NB = D / 32;   // 32-row d blocks of O^T
  constexpr int P = C::kLoadsPerWave;
  constexpr int NR = 2 * NB;   // transposed V reads per k-step of the PV product
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i32 = lane & 31, g2 = lane >> 5;
  // task fields and per-sequence scalars are wave-uniform; readfirstlane lets the compiler
  // keep everything derived from them (block ids, tile bounds, branches) in scalar registers
  const int s = __builtin_amdgcn_readfirstlane(t.seq);
  const int h = __builtin_amdgcn_readfirstlane(t.head);
  const int cu0 = __builtin_amdgcn_readfirstlane(a.cu_seqlens[s]);
  const int ql = __builtin_amdgcn_readfirstlane(a.cu_seqlens[s + 1]) - cu0;
  const int prefix = __builtin_amdgcn_readfirstlane(a.context_lens[s]) - ql;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int kvh = h / G;
  const int bs = a.block_size;
  const int r0 = __builtin_amdgcn_readfirstlane(t.q_row0);
  const int rows = __builtin_amdgcn_readfirstlane(t.q_rows);
  const int kv0 = __builtin_amdgcn_readfirstlane(t.kv0);
  const int kv1 = __builtin_amdgcn_readfirstlane(t.kv1);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int qi = r0 + 32 * wave + i32;              // this lane's query row (sequence-relative)
  const bool row_ok = qi < r0 + rows;
  const int wave_pos_lo = prefix + r0 + 32 * wave_u;  // position of the wave's first row
  const float c = a.scale_log2;

  bf16x8 qf[KS];
  {
    // CODES: k-step 2j takes d = 32j + 16*g2 + 0..7 and k-step 2j+1 d = 32j + 16*g2 + 8..15,
    // the order in which a K read returns a key's codes
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         (static_cast<size_t>(cu0 + qi) * a.num_q_heads + h) * D +
                         (CODES ? 16 : 8) * g2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row_ok)
        v = *reinterpret_cast<const u32x4*>(qp + (CODES ? 32 * (ks >> 1) + 8 * (ks & 1) : 16 * ks));
      qf[ks] = as_bf16x8(v);
    }
  }

  constexpr int EB = FP8 || CODES ? 1 : 2;  // bytes per element in the pages
  const size_t head_stride = static_cast<size_t>(bs) * D;
  const size_t block_stride = static_cast<size_t>(a.num_kv_heads) * head_stride;
  const char* kbase = static_cast<const char*>(a.k_pages) + kvh * head_stride * EB;
  const char* vbase = static_cast<const char*>(a.v_pages) + kvh * head_stride * EB;
  cint32* bt = (cint32*)(a.block_table + static_cast<size_t>(s) * a.max_blocks);

  // ---- LDS: [K buffer 0 | K buffer 1 | V buffer 0 | V buffer 1], one 64-key tile each.
  // Lane-constant addresses point into buffer 0 of each kind; buffer, key block and k-step
  // enter as instruction offsets.
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem));
  // K row i32, chunk 2*ks + g2. The row base is a multiple of 256 bytes and k-step ks only
  // flips chunk bits 1..3, so the address of k-step ks is ka0 ^ (ks << 5).
  uint32_t ka0 = lds0 + i32 * C::kRowBytes + ((g2 ^ lds_swz<D, CODES>(i32)) << 4);
  const int gq = lane >> 4, jq = lane & 15;
  const int v_key = 4 * g2 + (jq >> 2);     // key of this lane's segment (+ 16*kk, + 8)
  const int v_d = 16 * (gq & 1) + 4 * (jq & 3);
  uint32_t va[2 * NB];                      // [2n + half]: d block n, keys +8*half
#pragma unroll
  for (int n = 0; n < NB; ++n)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int key = v_key + 8 * hf;
      va[2 * n + hf] = lds0 + 2 * C::kTileBytes + key * C::kRowBytes +
                       ((((32 * n + v_d) >> 3) ^ lds_swz<D>(key)) << 4) + 8 * (jq & 1);
    }
  // CODES: transposed V reads of codes. Byte b of lane i32 + 32*g2's result must be the key of
  // its k-slot b in the P operand, 4*g2 + b%4 + 8*(b/4) (+ 16*kk: the keys the score layout gives
  // that lane), at d = 32n + i32. Lane j of a 16-lane group receives its byte b from the
  // segment of lane 2b + j/8, so lane (gq, jq) addresses key 4*(gq/2) + (jq/2)%4 + 8*(jq/8) at
  // d = 32n + 16*(gq%2) + 8*(jq%2): the V^T operand of d block n and k-step kk.
  uint32_t vca[NB] = {};
  if constexpr (CODES) {
    const int key = 4 * (gq >> 1) + ((jq >> 1) & 3) + 8 * (jq >> 3);
#pragma unroll
    for (int n = 0; n < NB; ++n)
      vca[n] = lds0 + 2 * C::kTileBytes + key * C::kRowBytes +
               (((2 * n + (gq & 1)) ^ lds_swz<D, true>(key)) << 4) + 8 * (jq & 1);
  }
  // ---- direct-load addressing. Each wave loads 16 consecutive keys of every tile
  // (P pieces of kKeysPerLoad keys). Tiles start at multiples of 64 keys and blocks hold at
  // least 16 keys, so those 16 keys lie in one block: one wave-uniform block id per tile (a
  // scalar load through the constant address space). Within the block the key's slot is
  // (ts & (bs-1)) + (key_in_tile & (bs-1)), so the lane part of the offset is constant.
  // Piece i of a wave starts kKeysPerLoad*i keys (1 KiB) after piece 0 and the swizzle of its
  // keys differs from piece 0's in the low chunk bits only: its lane offset is
  // (dma0 ^ (swizzle difference << 4)) + 1024*i, the last term an instruction offset.
  const int key0 = wave_u * P * C::kKeysPerLoad + lane / C::kChunks;
  uint32_t dma0 = (key0 & (bs - 1)) * C::kRowBytes +
                        (((lane % C::kChunks) ^ lds_swz<D, CODES>(key0)) << 4);
  auto dma_off = [&](int i) -> uint32_t {
    return dma0 ^
           ((lds_swz<D, CODES>(key0 + i * C::kKeysPerLoad) ^ lds_swz<D, CODES>(key0)) << 4);
  };
  // The pieces' lane offsets within a tile, dma_off(i) + 1024*i (fp8: half of it, the offset of
  // the same elements' codes), computed once and held across the loop (P registers): each load
  // of a full tile then takes the tile's block address as a scalar base and its own
  // never-rewritten offset register. Addresses rebuilt before every load in one register make
  // each load wait until the previous one has read it.
  uint32_t dmo[P];
#pragma unroll
  for (int i = 0; i < P; ++i) dmo[i] = FP8 ? (dma_off(i) + i * 1024) / 2 : dma_off(i) + i * 1024;
  const int ntiles = (kv1 - kv0 + C::kTile - 1) / C::kTile;
  // block id of this wave's keys in tile `tile`; keys past the range are clamped, so any tile
  // number is safe
  auto block_id = [&](int tile) -> int {
    const int kp = min(kv0 + tile * C::kTile + wave_u * P * C::kKeysPerLoad, kv1 - 1);
    return bt[kp >> a.bs_shift];
  };
  // CODES: page scales of the four 16-key groups of tile `tile` (each group one wave's direct
  // loads, so one page), K (which 0) or V (1); clamped like the loads
  float ksc4[4], vsc4[4];
  auto tile_scales = [&](int tile, int which, float (&out)[4]) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int kp = min(kv0 + tile * C::kTile + 16 * g, kv1 - 1);
      const size_t page = static_cast<size_t>(bt[kp >> a.bs_shift]) * a.num_kv_heads + kvh;
      out[g] = ((cfloat*)a.scales)[2 * page + which];
    }
  };
  // fp8 staging: codes of the K (0) and V (1) pieces in flight, and their pages' scales
  u32x2 stage[2][P];
  float stage_sc[2] = {0.f, 0.f};
  // Keys past kv1 (last tile only) are read from key kv1-1 instead (valid memory, finite
  // values); they are masked in the scores. `which` 0 loads K into K buffer `buf`, 1 loads V.
  // The fp8 form of an element sits at half the byte offset of its bf16 form.
  auto issue = [&](int tile, int id, int which, int buf) {
    const int ts = kv0 + tile * C::kTile;
    const bool full = ts + C::kTile <= kv1;
    const char* page = (which ? vbase : kbase) + static_cast<size_t>(id) * block_stride * EB;
    char* dst0 = smem + (2 * which + buf) * C::kTileBytes + wave_u * P * 1024;
    const uint32_t tile_slot = static_cast<uint32_t>(ts & (bs - 1)) * C::kRowBytes;
    if constexpr (FP8) {
      stage_sc[which] = ((cfloat*)a.scales)[2 * (static_cast<size_t>(id) * a.num_kv_heads + kvh) + which];
      if (full) {
        const char* base = page + tile_slot / 2;
#pragma unroll
        for (int i = 0; i < P; ++i) stage[which][i] = *reinterpret_cast<const u32x2*>(base + dmo[i]);
        asm volatile("");
      } else {
#pragma unroll
        for (int i = 0; i < P; ++i) {
          const int kabs = min(ts + key0 + i * C::kKeysPerLoad, kv1 - 1);
          stage[which][i] = *reinterpret_cast<const u32x2*>(
              page + (kabs & (bs - 1)) * (C::kRowBytes / 2) + (dmo[i] & (C::kRowBytes / 2 - 1)));
        }
      }
    } else if (full) {
      const char* base = page + tile_slot;
#pragma unroll
      for (int i = 0; i < P; ++i)
        __builtin_amdgcn_global_load_lds(base + dmo[i],
                                         (__attribute__((address_space(3))) void*)(dst0 + i * 1024),
                                         16, 0, 0);
      asm volatile("");  // keeps this path's last load from being merged with the partial path's
    } else {
#pragma unroll
      for (int i = 0; i < P; ++i) {
        const int kabs = min(ts + key0 + i * C::kKeysPerLoad, kv1 - 1);
        __builtin_amdgcn_global_load_lds(
            page + (kabs & (bs - 1)) * C::kRowBytes + (dmo[i] & (C::kRowBytes - 1)),
            (__attribute__((address_space(3))) void*)(dst0 + i * 1024), 16, 0, 0);
      }
    }
  };
  // fp8: converts the staged codes of piece i of `which` and writes them to LDS buffer `buf`,
  // each lane at the position its direct load would have written (16 bytes per lane)
  auto commit_piece = [&](int which, int buf, int i) {
    if constexpr (FP8) {
      char* dst = smem + (2 * which + buf) * C::kTileBytes + wave_u * P * 1024 + 16 * lane;
      const float sc = stage_sc[which];
      const u32x2 w = stage[which][i];
      *reinterpret_cast<u32x4*>(dst + i * 1024) =
          u32x4{fp8x2_to_bf16x2<false>(w[0], sc), fp8x2_to_bf16x2<true>(w[0], sc),
                fp8x2_to_bf16x2<false>(w[1], sc), fp8x2_to_bf16x2<true>(w[1], sc)};
    }
  };
  auto commit = [&](int which, int buf) {
#pragma unroll
    for (int i = 0; i < P; ++i) commit_piece(which, buf, i);
  };
  // fp8: a barrier that waits for this wave's LDS operations only (lgkmcnt; vmcnt and expcnt
  // not waited for), so register loads stay in flight; the empty asm statements keep the
  // compiler from moving LDS accesses across it
  auto lds_barrier = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  f32x16 acc[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[n][r] = 0.f;
  float m = -INFINITY, l = 0.f;

  // tiles this wave computes: those with a key at or before its last row's position
  int nw = 0;
  if (32 * wave_u < rows) {
    const int last = wave_pos_lo + 31;     // keys <= last are visible to some row of the wave
    nw = last < kv0 ? 0 : min(ntiles, (last - kv0) / C::kTile + 1);
  }
  nw = __builtin_amdgcn_readfirstlane(nw);

  // ---- the three pieces of work on a tile. The loop runs them software-pipelined: the
  // scores of tile j+1 are computed while the exponentials of tile j are formed, and the
  // value product of tile j runs while the causal mask of tile j+1 is applied, so the matrix
  // cores and the vector ALUs work on independent data inside one wave. Each matrix
  // instruction is followed by its share of the vector work, and sched_barrier keeps that
  // order: the scheduler would otherwise gather all exponentials in one place.
  //
  // Reference maximum. The exponentials of a tile are taken against the running reference m
  // without first taking the tile's maximum: only the wave's first tile sets m from its exact
  // maximum. Each lane sums its tile's weights (the bf16-rounded values the value product
  // uses, so numerator and denominator use the same weights); a sum above 2^16 (or an
  // infinite one) bounds every weight of that lane only loosely, so the wave then takes the
  // tile's true maximum, rescales acc and l to it and forms the exponentials again. Otherwise
  // every weight is at most 2^16 and the result is the same softmax with another reference.
  // Rows with a visible key in the first tile have l >= 1 from then on, so later tiles far
  // below m only lose what fp32 would lose anyway.
  u32x4 pw[4];                              // P of the current tile, bf16, per PV k-step
  // Phase A: scores of the next tile (K buffer KB) into sn; exponentials of sc into pw, their
  // sum into psum.
  auto phase_a = [&](auto kb_tag, auto do_qk, auto do_exp, f32x16 (&sn)[2], f32x16 (&sc)[2],
                     float& psum) {
    constexpr int KOFF = decltype(kb_tag)::value * C::kTileBytes;
    constexpr bool QK = decltype(do_qk)::value, EXP = decltype(do_exp)::value;
    const float muse = m == -INFINITY ? 0.f : m;
    float ps0 = 0.f, ps1 = 0.f;
    float ep0 = 0.f, ep1 = 0.f;             // exponentials of the previous word
    // packs the exponentials of word w (held in ep0, ep1) and adds them to a partial sum
    auto pack_word = [&](int w) {
      uint32_t word = pack_bf16x2(ep0, ep1);
      // pins the word here: without it the packing sinks towards its first use in the value
      // product, after the matrix steps it is meant to overlap
      asm volatile("" : "+v"(word));
      pw[w >> 2][w & 3] = word;
      const bf16x2 one2 = __builtin_bit_cast(bf16x2, 0x3f803f80u);
      if (w & 1)
        ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, word), one2, ps1, false);
      else
        ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, word), one2, ps0, false);
    };
    // word w of pw (0..15): exponentials of scores 2w, 2w+1 of key block w / 8. The previous
    // word is packed after these exponentials are issued, so no packing waits on a
    // transcendental result.
    auto exp_word = [&](int w) {
      const int kb = w >> 3, r = 2 * (w & 7);
      const float e0 = fast_exp2(fmaf(sc[kb][r], c, -muse));
      const float e1 = fast_exp2(fmaf(sc[kb][r + 1], c, -muse));
      if (w > 0) pack_word(w - 1);
      ep0 = e0;
      ep1 = e1;
    };
    if constexpr (QK) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sn[kb][r] = 0.f;
    }
    // four matrix steps on key block KB_, k-steps KS0..KS0+3 from kw, each followed by one
    // word of exponentials (words W0..W0+3)
    // (`step(q)`, CODES: the conversion of one operand of the next group, beside matrix step q)
    auto group = [&](f32x16& acc_s, const u32x4 (&kw)[4], int ks0, int w0, auto step) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (QK)
          acc_s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kw[q]), qf[ks0 + q], acc_s, 0, 0, 0);
        if constexpr (EXP) exp_word(w0 + q);
        step(q);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    auto none = [](int) {};
    u32x4 k0[4], k1[4];
    if constexpr (CODES) {
      // read j of key block kb: the 16 codes of k-steps 2j and 2j+1 of key i32 + 32kb, taken
      // times the scale of the key's page (keys 0-15 and 16-31 of a block lie in two groups)
      const float sk0 = i32 < 16 ? ksc4[0] : ksc4[1];
      const float sk1 = i32 < 16 ? ksc4[2] : ksc4[3];
      const uint32_t kc[4] = {ka0, ka0 ^ (1u << 5), ka0 ^ (2u << 5), ka0 ^ (3u << 5)};
      // operand q of a group: the low (q even) or high (q odd) 8 codes of read q/2 of the pair
      auto conv1 = [&](const u32x4& cw, bool hi, float sc) -> u32x4 {
        const uint32_t w0 = hi ? cw[2] : cw[0], w1 = hi ? cw[3] : cw[1];
        return u32x4{fp8x2_to_bf16x2<false>(w0, sc), fp8x2_to_bf16x2<true>(w0, sc),
                     fp8x2_to_bf16x2<false>(w1, sc), fp8x2_to_bf16x2<true>(w1, sc)};
      };
      // two operand sets used in turn: the next group's operands are converted one per matrix
      // step of the current group
      u32x4 kwa[4], kwb[4];
      if constexpr (QK) {
        ds_read_b128_x4_issue<KOFF>(kc, k0);
        ds_read_b128_x4_issue<KOFF + 32 * C::kRowBytes>(kc, k1);
        lds_wait<4>(k0);
#pragma unroll
        for (int q = 0; q < 4; ++q) kwa[q] = conv1(k0[q >> 1], q & 1, sk0);
      }
      group(sn[0], kwa, 0, 0, [&](int q) {
        if constexpr (QK) kwb[q] = conv1(k0[2 + (q >> 1)], q & 1, sk0);
      });
      if constexpr (QK) lds_wait<0>(k1);
      group(sn[0], kwb, 4, 4, [&](int q) {
        if constexpr (QK) kwa[q] = conv1(k1[q >> 1], q & 1, sk1);
      });
      group(sn[1], kwa, 0, 8, [&](int q) {
        if constexpr (QK) kwb[q] = conv1(k1[2 + (q >> 1)], q & 1, sk1);
      });
      group(sn[1], kwb, 4, 12, none);
    } else if constexpr (KS == 8) {
      const uint32_t kl[4] = {ka0, ka0 ^ (1u << 5), ka0 ^ (2u << 5), ka0 ^ (3u << 5)};
      const uint32_t kh[4] = {ka0 ^ (4u << 5), ka0 ^ (5u << 5), ka0 ^ (6u << 5), ka0 ^ (7u << 5)};
      if constexpr (QK) {
        ds_read_b128_x4_issue<KOFF>(kl, k0);
        ds_read_b128_x4_issue<KOFF>(kh, k1);
        lds_wait<4>(k0);
      }
      group(sn[0], k0, 0, 0, none);
      if constexpr (QK) {
        ds_read_b128_x4_issue<KOFF + 32 * C::kRowBytes>(kl, k0);
        lds_wait<4>(k1);
      }
      group(sn[0], k1, 4, 4, none);
      if constexpr (QK) {
        ds_read_b128_x4_issue<KOFF + 32 * C::kRowBytes>(kh, k1);
        lds_wait<4>(k0);
      }
      group(sn[1], k0, 0, 8, none);
      if constexpr (QK) lds_wait<0>(k1);
      group(sn[1], k1, 4, 12, none);
    } else {
      const uint32_t kl[4] = {ka0, ka0 ^ (1u << 5), ka0 ^ (2u << 5), ka0 ^ (3u << 5)};
      if constexpr (QK) {
        ds_read_b128_x4_issue<KOFF>(kl, k0);
        ds_read_b128_x4_issue<KOFF + 32 * C::kRowBytes>(kl, k1);
        lds_wait<4>(k0);
      }
      group(sn[0], k0, 0, 0, none);
      if constexpr (QK) lds_wait<0>(k1);
      group(sn[1], k1, 0, 4, none);
      if constexpr (EXP) {
#pragma unroll
        for (int w = 8; w < 16; ++w) exp_word(w);
      }
    }
    if constexpr (EXP) {
      pack_word(15);
      psum = ps0 + ps1;
    }
  };
  // The slow path of the reference maximum: the true maximum of the scores sc of the current
  // tile becomes the reference (when above m), acc and l are rescaled to it and the
  // exponentials and their sum are formed again.
  auto retake = [&](f32x16 (&sc)[2], float& psum) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
    mx = fmaxf(mx, wave_shfl_xor(mx, 32)) * c;
    const float mnew = fmaxf(m, mx);
    const float alpha = mnew == -INFINITY ? 1.f : fast_exp2(m - mnew);
    l *= alpha;
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[n] *= alpha;
    m = mnew;
    const float muse = m == -INFINITY ? 0.f : m;
    float ps = 0.f;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int kb = w >> 3, r = 2 * (w & 7);
      const uint32_t word = pack_bf16x2(fast_exp2(fmaf(sc[kb][r], c, -muse)),
                                        fast_exp2(fmaf(sc[kb][r + 1], c, -muse)));
      pw[w >> 2][w & 3] = word;
      ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, word),
                                           __builtin_bit_cast(bf16x2, 0x3f803f80u), ps, false);
    }
    psum = ps;
  };
  // Phase B: value product of the current tile (V buffer VB) with pw, and the causal mask of
  // the next tile's scores sn (starting at key ts_next); with MAX also the maximum of sn and
  // the rescale to it (the wave's first tile only).
  // `hook(kk)` runs after the matrix steps of k-step kk (fp8: a share of the tile conversions).
  auto phase_b = [&](auto vb_tag, auto do_pv, auto do_max, f32x16 (&sn)[2], int ts_next,
                     auto hook) {
    constexpr int VOFF = decltype(vb_tag)::value * C::kTileBytes;
    constexpr bool PV = decltype(do_pv)::value, MAX = decltype(do_max)::value;
    constexpr int NV = CODES ? NB : NR;     // reads per k-step batch
    typedef u32x2 VR[NV];
    VR vr0, vr1;
    auto v_issue = [&](auto kk_tag, VR& r) {
      constexpr int KK = decltype(kk_tag)::value;
      if constexpr (CODES)
        ds_read_b64_tr_b8_x4_issue<VOFF + 16 * KK * C::kRowBytes>(vca, r);
      else if constexpr (NR == 8)
        ds_read_b64_tr_b16_x8_issue<VOFF + 16 * KK * C::kRowBytes>(va, r);
      else
        ds_read_b64_tr_b16_x4_issue<VOFF + 16 * KK * C::kRowBytes>(va, r);
    };
    float mx = -INFINITY;
    if (ts_next + C::kTile - 1 > wave_pos_lo || ts_next + C::kTile > kv1) {
      // score (kb, r) holds key ts_next + 4*g2 + off with off = 32kb + 8(r/4) + r%4; it is
      // visible iff key < min(kv1, pos + 1), i.e. off < lim
      const int lim = min(kv1, prefix + qi + 1) - ts_next - 4 * g2;
      mask_block<0>(sn[0], lim);
      mask_block<32>(sn[1], lim);
    }
    // k-step kk: NB matrix steps, each followed by the maximum over a share of sn
    constexpr int kMaxPer = 32 / (4 * NB);  // scores folded per matrix step
    auto pv = [&](int kk, VR& r) {
      const bf16x8 pf = as_bf16x8(pw[kk]);
      // CODES: keys 16kk + 0..15 lie in group kk, one page scale for the k-step; the operand of
      // matrix step n+1 is converted beside step n
      const float sv = CODES ? vsc4[kk] : 0.f;
      auto vconv = [&](int n) -> u32x4 {
        return u32x4{fp8x2_to_bf16x2<false>(r[n][0], sv), fp8x2_to_bf16x2<true>(r[n][0], sv),
                     fp8x2_to_bf16x2<false>(r[n][1], sv), fp8x2_to_bf16x2<true>(r[n][1], sv)};
      };
      u32x4 vnext;
      if constexpr (CODES && PV) vnext = vconv(0);
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        if constexpr (PV) {
          u32x4 vw;
          if constexpr (CODES)
            vw = vnext;
          else
            vw = u32x4{r[2 * n][0], r[2 * n][1], r[2 * n + 1][0], r[2 * n + 1][1]};
          acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vw), pf, acc[n], 0, 0, 0);
          if constexpr (CODES)
            if (n + 1 < NB) vnext = vconv(n + 1);
        }
        if constexpr (MAX) {
#pragma unroll
          for (int i = 0; i < kMaxPer; ++i) {
            const int v = (kk * NB + n) * kMaxPer + i;
            mx = fmaxf(mx, sn[v >> 4][v & 15]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if constexpr (PV) {
      v_issue(std::integral_constant<int, 0>(), vr0);
      v_issue(std::integral_constant<int, 1>(), vr1);
      lds_wait<NV>(vr0);
    }
    pv(0, vr0);
    hook(0);
    if constexpr (PV) {
      v_issue(std::integral_constant<int, 2>(), vr0);
      lds_wait<NV>(vr1);
    }
    pv(1, vr1);
    hook(1);
    if constexpr (PV) {
      v_issue(std::integral_constant<int, 3>(), vr1);
      lds_wait<NV>(vr0);
    }
    pv(2, vr0);
    hook(2);
    if constexpr (PV) lds_wait<0>(vr1);
    pv(3, vr1);
    hook(3);
    if constexpr (MAX) {
      // the first tile: its exact maximum becomes the reference (acc and l are still zero)
      m = fmaxf(mx, wave_shfl_xor(mx, 32)) * c;
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using T_ = std::true_type;
  using F_ = std::false_type;

  // ---- prologue: K0, V0 into buffers 0, K1 into K buffer 1; scores and maximum of tile 0
  f32x16 sa[2], sb[2];
  {
    const int id0 = block_id(0);
    issue(0, id0, 0, 0);
    issue(0, id0, 1, 0);
    commit(0, 0);
    commit(1, 0);
  }
  int idV = block_id(1);                    // tile j+1 (its V is loaded in iteration j)
  if (ntiles > 1) {
    issue(1, idV, 0, 1);
    commit(0, 1);
  }
  int idK = block_id(2);                    // tile j+2 (its K is loaded in iteration j)
  int idN = block_id(3);                    // tile j+3, read one iteration ahead
  if constexpr (FP8) {
    // the codes iteration 0 converts: K(2) and V(1)
    if (ntiles > 2) issue(2, idK, 0, 0);
    if (ntiles > 1) issue(1, idV, 1, 0);
    lds_barrier();
  } else {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if constexpr (CODES) tile_scales(0, 0, ksc4);
  if (nw > 0) {
    float unused;
    phase_a(I0(), T_(), F_(), sa, sb, unused);
    phase_b(I0(), F_(), T_(), sa, kv0, [](int) {});
  }

  // ---- iteration j: wait for K(j+1) and V(j); load K(j+2) and V(j+1) into the buffers the
  // previous iteration finished with; exponentials of j with scores of j+1; value product
  // of j with the mask of j+1. Unrolled by two so buffers and score sets are named
  // statically: even j reads K buffer 1, V buffer 0, keeps scores of j in sa.
  //
  // Buffer protocol. K(t) lives in K buffer t%2: its direct loads are issued in iteration t-2
  // and it is read in iteration t-1 (tile 0: loaded and read in the prologue); V(t) lives in V
  // buffer t%2, loaded in iteration t-1 and read in iteration t. Every wave passes the
  // barrier at the top of an iteration only after s_waitcnt(0), i.e. after its own direct
  // loads have written LDS (vmcnt) and its own LDS reads have returned their data (lgkmcnt).
  // So once any wave is past the barrier of iteration j, (a) all loads issued before it are
  // in LDS for every wave, and (b) every read issued before it is complete, and a buffer read
  // in iteration j-1 can be overwritten. Iteration 0 overwrites K buffer 0, whose tile 0 the
  // prologue read, so it needs that barrier too whenever it issues K(2) (a wave with no tile
  // to compute skips the prologue's reads and would otherwise reach the issue first).
  //
  // fp8 pages: the buffers and their reads are the same; what changes is how a tile gets
  // there. The codes of K(t) are loaded into registers at the end of iteration t-3 (for t = 2:
  // in the prologue) and converted and written to K buffer t%2 during the value product of
  // iteration t-2; those of V(t) are loaded at the end of iteration t-2 and written during
  // iteration t-1. These are ordinary LDS writes, so a wave passes the barrier after
  // s_waitcnt lgkmcnt(0) alone: its writes are in LDS (a) and its reads have returned (b), while
  // its register loads for the next conversions stay in flight across the barrier.
  auto iteration = [&](int j, auto par_tag, f32x16 (&scur)[2], f32x16 (&snext)[2]) {
    constexpr int PAR = decltype(par_tag)::value;
    // opaque redefinition: values derived from these bases (the per-k-step and per-piece
    // addresses) are then recomputed where used instead of held in registers across the loop
    asm volatile("" : "+v"(ka0));
    // the offsets stay 32-bit values in their own registers, so each load can take them as its
    // offset operand next to the scalar base
#pragma unroll
    for (int i = 0; i < P; ++i) asm volatile("" : "+v"(dmo[i]));
    if constexpr (CODES) {
      // page scales of the tiles this iteration reads: K(j+1), V(j) (scalar loads, ahead of
      // the barrier's wait)
      tile_scales(j + 1, 0, ksc4);
      tile_scales(j, 1, vsc4);
    }
    if (j > 0 || ntiles > 2) {
      if constexpr (FP8) {
        lds_barrier();
      } else {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
    }
    if constexpr (!FP8) {
      if (j + 2 < ntiles) issue(j + 2, idK, 0, PAR);
      if (j + 1 < ntiles) issue(j + 1, idV, 1, 1 - PAR);
    }
    idV = idK;
    idK = idN;
    idN = block_id(j + 4);
    // fp8: K(j+2) and V(j+1), staged in registers, go to their buffers in shares after the
    // value product's k-steps (P/2 pieces each), or all at once on a wave with nothing to
    // compute
    const bool k_due = j + 2 < ntiles, v_due = j + 1 < ntiles;
    auto convert_share = [&](int kk) {
      if constexpr (FP8) {
#pragma unroll
        for (int q = 0; q < P / 2; ++q) {
          const int item = kk * (P / 2) + q;
          const int which = item / P, i = item % P;
          if (which == 0 ? k_due : v_due) commit_piece(which, which ? 1 - PAR : PAR, i);
        }
      }
    };
    // The scores of tile j+1 are formed even when this wave has no key to see there (its
    // last tile, or past the range): the mask then sets all of them to -inf, whatever the K
    // buffer holds, and their weights are zero. One code path keeps the accumulators in
    // place across the loop.
    if (j < nw) {
      float psum;
      phase_a(std::integral_constant<int, 1 - PAR>(), T_(), T_(), snext, scur, psum);
      if (__builtin_amdgcn_ballot_w64(!(psum <= 65536.f)) != 0) retake(scur, psum);
      l += psum;
      phase_b(std::integral_constant<int, PAR>(), T_(), F_(), snext, kv0 + (j + 1) * C::kTile,
              convert_share);
    } else if constexpr (FP8) {
      if (k_due) commit(0, PAR);
      if (v_due) commit(1, 1 - PAR);
    }
    if constexpr (FP8) {
      // the codes the next iteration converts: K(j+3) and V(j+2)
      if (j + 3 < ntiles) issue(j + 3, idK, 0, 0);
      if (j + 2 < ntiles) issue(j + 2, idV, 1, 0);
    }
  };
  for (int j = 0; j < ntiles; j += 2) {
    iteration(j, I0(), sa, sb);
    if (j + 1 >= ntiles) break;
    iteration(j + 1, I1(), sb, sa);
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

// AHEAD: each wave keeps two chunks of page reads in flight (two waves per SIMD) instead of one
// (three waves per SIMD); measured faster on decode tables, slower on shared-prefix ones.
template <typename T, int D, bool AHEAD>
__global__ __launch_bounds__(kThreads, AHEAD ? 2 : 3) void decode_kernel(AttnArgs a) {
  __shared__ float smem[kMergeFloats<D>];
  const pa_task t = a.tasks[blockIdx.x];
  if (t.kind != PA_TASK_DECODE && t.kind != PA_TASK_SHARED) return;
  if constexpr (sizeof(T) == 2)
    decode_task_bf16<D, AHEAD, true>(a, t, smem);
  else
    decode_task_f32<D>(a, t, smem);
}

template <int D>
__global__ __launch_bounds__(kThreads) void decode_fp8_kernel(AttnArgs a) {
  __shared__ float smem[kMergeFloats<D>];
  const pa_task t = a.tasks[blockIdx.x];
  // verify tasks need the packed rows' offsets (cu_seqlens), which only the verify entry passes;
  // shared-prefix tasks address their members' rows as consecutive decode rows (no cu_seqlens)
  if (t.kind == PA_TASK_PREFILL || (t.kind == PA_TASK_VERIFY && !a.cu_seqlens) ||
      (t.kind == PA_TASK_SHARED && a.cu_seqlens))
    return;
  decode_task_fp8<D, true>(a, t, smem);
}

// a.stream_reads: the table holds no prefill tiles, so the decode tasks' page streams have nothing
// reused in the caches to protect (non-temporal reads measured faster there, and slower beside
// prefill tiles)
template <int D>
__global__ __launch_bounds__(kThreads, 2) void meta_attn_kernel(AttnArgs a) {
  constexpr size_t kPrefill = PrefillCfg<D>::kSmemBytes;
  constexpr size_t kDecode = kMergeFloats<D> * sizeof(float);
  __shared__ __attribute__((aligned(1024))) char smem[kPrefill > kDecode ? kPrefill : kDecode];
  const pa_task t = a.tasks[xcd_remap(blockIdx.x, a.num_tasks)];
  if (t.kind == PA_TASK_PREFILL)
    prefill_task<D>(a, t, smem);
  else if (a.stream_reads)
    decode_task_bf16<D, true, true>(a, t, reinterpret_cast<float*>(smem));
  else
    decode_task_bf16<D, true, false>(a, t, reinterpret_cast<float*>(smem));
}

// The unified launch over fp8 pages: every task kind, rows addressed through cu_seqlens.
template <int D>
__global__ __launch_bounds__(kThreads, 2) void meta_attn_fp8_kernel(AttnArgs a) {
  // D = 128: codes in LDS, converted at the operand reads; D = 64: converted on the way in
  constexpr int kMode = D == 128 ? 2 : 1;
  constexpr size_t kPrefill = PrefillCfg<D, kMode == 2>::kSmemBytes;
  constexpr size_t kDecode = kMergeFloats<D> * sizeof(float);
  __shared__ __attribute__((aligned(1024))) char smem[kPrefill > kDecode ? kPrefill : kDecode];
  const pa_task t = a.tasks[xcd_remap(blockIdx.x, a.num_tasks)];
  if (t.kind == PA_TASK_PREFILL)
    prefill_task<D, kMode>(a, t, smem);
  else if (a.stream_reads)
    decode_task_fp8<D, true>(a, t, reinterpret_cast<float*>(smem));
  else
    decode_task_fp8<D, false>(a, t, reinterpret_cast<float*>(smem));
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

// Cache write into fp8 pages (cann-recipes-infer page, section 5.2: values are scaled before
// they are stored and each page keeps its scale). A page that this step writes into is
// rescaled as a whole: its
// valid rows -- the ones cached before (code * old scale, exact in fp32) and this step's rows
// (bf16) -- set the page maximum, the new scale is the smallest power of two 2^k (k >= -120)
// with max <= 448 * 2^k, and every valid row is encoded again as the round-to-nearest-even
// E4M3FN code of value * 2^-k (an exact scaling). Rows past the context stay untouched.
// Grid: x = runs of `tokens_per_group` consecutive packed tokens, y = groups of four (tensor,
// kv head) units, one wave per unit. A page is rewritten by the wave that meets the first new
// row of its block, so each touched page is rewritten by exactly one wave; a wave walks its run
// from one block's first row to the next, so runs of prefill tokens cost one step per page,
// not per token. Two passes over the page: the maximum, then the codes; each lane reads and
// writes the same eight codes in both, and the new codes and scale depend on the maximum over
// all lanes' reads, so no write precedes a read of the old page.
template <int D>
__device__ void rewrite_fp8_page(const __bf16* k_new, const __bf16* v_new, uint8_t* k_pages,
                                 uint8_t* v_pages, float* scales, const int32_t* block_table,
                                 int32_t max_blocks, int32_t num_kv_heads, int32_t block_size,
                                 int32_t bs_shift, int unit, int s, int c0, int ctx, int P,
                                 int pos) {
  const int lb = pos >> bs_shift;
  const int row0 = lb << bs_shift;                          // position of the block's slot 0
  const int n_valid = min(ctx, row0 + block_size) - row0;
  const int n_old = pos - row0;                             // rows cached before this step
  const int blk = block_table[static_cast<size_t>(s) * max_blocks + lb];
  const int lane = threadIdx.x & 63;
  const int which = unit >= num_kv_heads;                   // 0: K, 1: V
  const int g = unit - which * num_kv_heads;
  uint8_t* codes = (which ? v_pages : k_pages) +
                   (static_cast<size_t>(blk) * num_kv_heads + g) * block_size * D;
  float* scale_p = scales + 2 * (static_cast<size_t>(blk) * num_kv_heads + g) + which;
  const __bf16* src = (which ? v_new : k_new) + g * D;
  const int64_t tok_p = static_cast<int64_t>(c0) - P;     // packed token of position 0
  const float old_scale = n_old > 0 ? *scale_p : 1.f;
  constexpr int Q8 = D / 8;                                 // eight-code groups per row
  const int groups = n_valid * Q8;
  // values of group e (row e / Q8, d = 8 * (e % Q8) + 0..7)
  auto load8 = [&](int e, float (&x)[8]) {
    const int j = e / Q8, q = e - j * Q8;
    if (j < n_old) {
      const u32x2 w = *reinterpret_cast<const u32x2*>(codes + j * D + 8 * q);
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int c = static_cast<int>(w[h >> 1]);
        const f32x2 v = (h & 1) ? __builtin_amdgcn_cvt_pk_f32_fp8(c, true)
                                : __builtin_amdgcn_cvt_pk_f32_fp8(c, false);
        x[2 * h] = v[0] * old_scale;
        x[2 * h + 1] = v[1] * old_scale;
      }
    } else {
      // position row0 + j is a new row: packed token cu[s] + (row0 + j - P)
      const u32x4 w = *reinterpret_cast<const u32x4*>(
          src + static_cast<size_t>(tok_p + row0 + j) * num_kv_heads * D + 8 * q);
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        x[2 * h] = __builtin_bit_cast(float, w[h] << 16);
        x[2 * h + 1] = __builtin_bit_cast(float, w[h] & 0xffff0000u);
      }
    }
  };
  float amax = 0.f;
  for (int e = lane; e < groups; e += 64) {
    float x[8];
    load8(e, x);
#pragma unroll
    for (int u = 0; u < 8; ++u) amax = fmaxf(amax, fabsf(x[u]));
  }
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) amax = fmaxf(amax, wave_shfl_xor(amax, sh));
  int k = 0;
  if (amax > 0.f) {
    const int e2 = ilogbf(amax);                            // 2^e2 <= amax < 2^(e2+1)
    k = amax <= ldexpf(1.75f, e2) ? e2 - 8 : e2 - 7;        // 448 * 2^(e2-8) = 1.75 * 2^e2
    k = max(k, -120);
  }
  for (int e = lane; e < groups; e += 64) {
    float x[8];
    load8(e, x);
    u32x2 w;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int c = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(x[4 * h], -k), ldexpf(x[4 * h + 1], -k), 0,
                                              false);
      c = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(x[4 * h + 2], -k), ldexpf(x[4 * h + 3], -k), c,
                                          true);
      w[h] = static_cast<uint32_t>(c);
    }
    const int j = e / Q8, q = e - j * Q8;
    *reinterpret_cast<u32x2*>(codes + j * D + 8 * q) = w;
  }
  if (lane == 0) *scale_p = ldexpf(1.f, k);
}

template <int D>
__global__ __launch_bounds__(kThreads) void reshape_and_cache_fp8_kernel(
    const __bf16* k_new, const __bf16* v_new, uint8_t* k_pages, uint8_t* v_pages,
    float* scales, const int32_t* block_table, int32_t max_blocks,
    const int32_t* cu_seqlens, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_tokens, int32_t tokens_per_group, int32_t num_kv_heads, int32_t block_size,
    int32_t bs_shift) {
  const int unit = blockIdx.y * (kThreads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (unit >= 2 * num_kv_heads) return;
  const int t0 = blockIdx.x * tokens_per_group;
  const int t1 = min(t0 + tokens_per_group, num_tokens);
  int lo_s = 0, hi_s = num_seqs;  // cu[lo_s] <= t0 < cu[hi_s]
  while (hi_s - lo_s > 1) {
    const int mid = (lo_s + hi_s) >> 1;
    if (cu_seqlens[mid] <= t0) lo_s = mid; else hi_s = mid;
  }
  int s = lo_s;
  for (int t = t0; t < t1 && s < num_seqs;) {
    const int c0 = cu_seqlens[s], c1 = cu_seqlens[s + 1];
    if (t >= c1) {
      ++s;
      continue;
    }
    const int ctx = context_lens[s];
    const int P = ctx - (c1 - c0);
    const int pos = P + (t - c0);
    // the first new row of its block: this wave rewrites the page
    if (pos == P || (pos & (block_size - 1)) == 0)
      rewrite_fp8_page<D>(k_new, v_new, k_pages, v_pages, scales, block_table, max_blocks,
                          num_kv_heads, block_size, bs_shift, unit, s, c0, ctx, P, pos);
    // the next block's first row, or the next sequence's first token
    t = min(t + ((pos | (block_size - 1)) + 1) - pos, c1);
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

int check_attn_shape(const char* who, int32_t num_seqs, int32_t hq, int32_t hkv, int32_t d,
                     int32_t bs, int32_t dtype, int32_t num_tasks, int32_t num_combines,
                     int32_t num_partials, int32_t max_blocks) {
  if (num_seqs < 0 || num_tasks < 0 || num_combines < 0 || num_partials < 0 || max_blocks < 0)
    return pa::set_error(PA_ERR_SHAPE, "%s: negative size", who);
  if (num_tasks > pa::kMaxWorkgroups || num_combines > pa::kMaxWorkgroups)
    return pa::set_error(PA_ERR_SHAPE, "%s: %d tasks, %d combines: one launch takes at most %d",
                         who, num_tasks, num_combines, pa::kMaxWorkgroups);
  if (hq < 1 || hkv < 1 || hq % hkv)
    return pa::set_error(PA_ERR_SHAPE, "%s: Hq %d is not a positive multiple of Hkv %d", who, hq, hkv);
  if (hq / hkv > pa::kMaxGroup)
    return pa::set_error(PA_ERR_SHAPE, "%s: Hq/Hkv = %d exceeds %d", who, hq / hkv, pa::kMaxGroup);
  if (!pa::head_dim_ok(d)) return pa::set_error(PA_ERR_SHAPE, "%s: head_dim %d not in {64, 128}", who, d);
  if (!pa::block_size_ok(bs))
    return pa::set_error(PA_ERR_BLOCK_SIZE, "%s: block_size %d is not a power of two in [16, 256]", who, bs);
  if (dtype != PA_BF16 && dtype != PA_FP32) return pa::set_error(PA_ERR_DTYPE, "%s: dtype %d", who, dtype);
  return PA_OK;
}

// The caller's workspace must hold every partial row whenever the table has partial rows or
// combine records.
int check_workspace(const char* who, int32_t num_partials, int32_t num_combines, int32_t d,
                    size_t ws_bytes, const void* ws) {
  if (num_partials > 0 || num_combines > 0) {
    if (!ws) return pa::set_error(PA_ERR_NULL, "%s: workspace is NULL", who);
    const size_t need = pa_workspace_bytes(num_partials, d);
    if (ws_bytes < need)
      return pa::set_error(PA_ERR_CAPACITY, "%s: workspace %zu bytes < %zu needed", who, ws_bytes, need);
  }
  return PA_OK;
}

int check_attn_scalars(const char* who, int32_t num_seqs, int32_t hq, int32_t hkv, int32_t d,
                       int32_t bs, int32_t dtype, int32_t num_tasks, int32_t num_combines,
                       int32_t num_partials, size_t ws_bytes, const void* ws, int32_t max_blocks) {
  if (int rc = check_attn_shape(who, num_seqs, hq, hkv, d, bs, dtype, num_tasks, num_combines,
                                num_partials, max_blocks))
    return rc;
  return check_workspace(who, num_partials, num_combines, d, ws_bytes, ws);
}

// The table's kind mask against the kinds this entry runs: a kind outside `allowed` would be
// skipped by the kernel and leave its rows of `out` unwritten, so it is refused here.
int check_kinds(const char* who, int32_t num_tasks, uint32_t kinds, uint32_t allowed) {
  if (num_tasks > 0 && kinds == 0)
    return pa::set_error(PA_ERR_INPUT, "%s: task_kinds is 0 for a table of %d tasks", who,
                         num_tasks);
  if (kinds & ~allowed)
    return pa::set_error(PA_ERR_INPUT, "%s: the table holds task kinds 0x%x; this entry runs 0x%x",
                         who, kinds, allowed);
  return PA_OK;
}

constexpr uint32_t kAllKinds = PA_KIND_BIT(PA_TASK_DECODE) | PA_KIND_BIT(PA_TASK_PREFILL) |
                               PA_KIND_BIT(PA_TASK_VERIFY) | PA_KIND_BIT(PA_TASK_SHARED);
constexpr uint32_t kDecodeKinds = PA_KIND_BIT(PA_TASK_DECODE) | PA_KIND_BIT(PA_TASK_SHARED);
constexpr uint32_t kVerifyKinds = PA_KIND_BIT(PA_TASK_DECODE) | PA_KIND_BIT(PA_TASK_VERIFY);

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
  a.scales = nullptr;
  a.max_blocks = max_blocks;
  a.num_q_heads = hq;
  a.num_kv_heads = hkv;
  a.block_size = bs;
  a.bs_shift = log2i(bs);
  a.num_tasks = num_tasks;
  a.scale_log2 = scale * kLog2e;
  a.stream_reads = 0;
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
  if (num_tokens > pa::kMaxWorkgroups)
    return pa::set_error(PA_ERR_SHAPE, "reshape_and_cache: %d tokens: one launch takes at most %d",
                         num_tokens, pa::kMaxWorkgroups);
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
                                 uint32_t task_kinds, const pa_combine* combines_dev,
                                 int32_t num_combines, int32_t num_partials, void* workspace,
                                 size_t workspace_bytes, void* out, void* stream) {
  if (int rc = check_attn_scalars("paged_attn_decode", num_seqs, num_q_heads, num_kv_heads,
                                  head_dim, block_size, dtype, num_tasks, num_combines,
                                  num_partials, workspace_bytes, workspace, max_blocks_per_seq))
    return rc;
  if (int rc = check_kinds("paged_attn_decode", num_tasks, task_kinds, kDecodeKinds)) return rc;
  if (num_tasks == 0) return pa::clear_error();
  if (!q || !k_pages || !v_pages || !block_table || !context_lens || !out || !tasks_dev ||
      (num_combines > 0 && !combines_dev))
    return pa::set_error(PA_ERR_NULL, "paged_attn_decode: NULL pointer");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const AttnArgs a = make_args(q, k_pages, v_pages, block_table, max_blocks_per_seq, nullptr,
                               context_lens, num_q_heads, num_kv_heads, head_dim, block_size,
                               scale, tasks_dev, num_tasks, num_partials, workspace, out);
  const bool ahead = !(task_kinds & PA_KIND_BIT(PA_TASK_SHARED));
  const dim3 grid(num_tasks), block(kThreads);
  if (dtype == PA_BF16) {
    if (head_dim == 128) {
      if (ahead)
        hipLaunchKernelGGL((decode_kernel<__bf16, 128, true>), grid, block, 0, st, a);
      else
        hipLaunchKernelGGL((decode_kernel<__bf16, 128, false>), grid, block, 0, st, a);
      launch_combine<__bf16, 128>(combines_dev, num_combines, nullptr, a, st);
    } else {
      if (ahead)
        hipLaunchKernelGGL((decode_kernel<__bf16, 64, true>), grid, block, 0, st, a);
      else
        hipLaunchKernelGGL((decode_kernel<__bf16, 64, false>), grid, block, 0, st, a);
      launch_combine<__bf16, 64>(combines_dev, num_combines, nullptr, a, st);
    }
  } else {
    if (head_dim == 128) {
      hipLaunchKernelGGL((decode_kernel<float, 128, false>), grid, block, 0, st, a);
      launch_combine<float, 128>(combines_dev, num_combines, nullptr, a, st);
    } else {
      hipLaunchKernelGGL((decode_kernel<float, 64, false>), grid, block, 0, st, a);
      launch_combine<float, 64>(combines_dev, num_combines, nullptr, a, st);
    }
  }
  return hip_check("paged_attn_decode");
}

namespace {

// The unified launch's checks that need no workspace: shapes, kinds, dtype, token count and the
// device pointers. PA_OK means the launch may be enqueued (given a workspace).
int varlen_checks(const char* who, const void* q, const void* k_pages, const void* v_pages,
                  const int32_t* block_table, int32_t max_blocks_per_seq,
                  const int32_t* cu_seqlens_q, const int32_t* context_lens, int32_t num_seqs,
                  int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                  int32_t head_dim, int32_t block_size, int32_t dtype, const pa_task* tasks_dev,
                  int32_t num_tasks, uint32_t task_kinds, const pa_combine* combines_dev,
                  int32_t num_combines, int32_t num_partials, const void* out) {
  if (int rc = check_attn_shape(who, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                dtype, num_tasks, num_combines, num_partials, max_blocks_per_seq))
    return rc;
  if (int rc = check_kinds(who, num_tasks, task_kinds, kAllKinds)) return rc;
  if (dtype != PA_BF16)
    return pa::set_error(PA_ERR_DTYPE, "%s: the MFMA path needs PA_BF16", who);
  if (num_tokens < num_seqs)
    return pa::set_error(PA_ERR_SHAPE, "%s: %d tokens for %d sequences", who, num_tokens,
                         num_seqs);
  if (num_tasks == 0) return PA_OK;
  if (!q || !k_pages || !v_pages || !block_table || !cu_seqlens_q || !context_lens || !out ||
      !tasks_dev || (num_combines > 0 && !combines_dev))
    return pa::set_error(PA_ERR_NULL, "%s: NULL pointer", who);
  return PA_OK;
}

// The unified launch and its combine, on `stream`, with partial rows in `workspace`.
int varlen_enqueue(const char* who, const void* q, const void* k_pages, const void* v_pages,
                   const int32_t* block_table, int32_t max_blocks_per_seq,
                   const int32_t* cu_seqlens_q, const int32_t* context_lens,
                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_size, float scale, const pa_task* tasks_dev, int32_t num_tasks,
                   const pa_combine* combines_dev, int32_t num_combines, int32_t num_partials,
                   uint32_t task_kinds, void* workspace, void* out, void* stream,
                   const float* scales = nullptr) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  AttnArgs a = make_args(q, k_pages, v_pages, block_table, max_blocks_per_seq, cu_seqlens_q,
                         context_lens, num_q_heads, num_kv_heads, head_dim, block_size, scale,
                         tasks_dev, num_tasks, num_partials, workspace, out);
  a.scales = scales;  // fp8 pages when set
  a.stream_reads = !(task_kinds & PA_KIND_BIT(PA_TASK_PREFILL));
  if (head_dim == 128) {
    if (scales)
      hipLaunchKernelGGL(meta_attn_fp8_kernel<128>, dim3(num_tasks), dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL(meta_attn_kernel<128>, dim3(num_tasks), dim3(kThreads), 0, st, a);
    launch_combine<__bf16, 128>(combines_dev, num_combines, cu_seqlens_q, a, st);
  } else {
    if (scales)
      hipLaunchKernelGGL(meta_attn_fp8_kernel<64>, dim3(num_tasks), dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL(meta_attn_kernel<64>, dim3(num_tasks), dim3(kThreads), 0, st, a);
    launch_combine<__bf16, 64>(combines_dev, num_combines, cu_seqlens_q, a, st);
  }
  return hip_check(who);
}

}  // namespace

extern "C" int paged_attn_varlen_prefill(
    const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
    int32_t max_blocks_per_seq, const int32_t* cu_seqlens_q, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, float scale, int32_t dtype, const pa_task* tasks_dev,
    int32_t num_tasks, uint32_t task_kinds, const pa_combine* combines_dev,
    int32_t num_combines, int32_t num_partials, void* workspace, size_t workspace_bytes,
    void* out, void* stream) {
  const char* who = "paged_attn_varlen_prefill";
  if (int rc = varlen_checks(who, q, k_pages, v_pages, block_table, max_blocks_per_seq,
                             cu_seqlens_q, context_lens, num_seqs, num_tokens, num_q_heads,
                             num_kv_heads, head_dim, block_size, dtype, tasks_dev, num_tasks,
                             task_kinds, combines_dev, num_combines, num_partials, out))
    return rc;
  if (int rc = check_workspace(who, num_partials, num_combines, head_dim, workspace_bytes,
                               workspace))
    return rc;
  if (num_tasks == 0) return pa::clear_error();
  return varlen_enqueue(who, q, k_pages, v_pages, block_table, max_blocks_per_seq, cu_seqlens_q,
                        context_lens, num_q_heads, num_kv_heads, head_dim, block_size, scale,
                        tasks_dev, num_tasks, combines_dev, num_combines, num_partials,
                        task_kinds, workspace, out, stream);
}

// Partial rows of paged_attn_varlen_prefill_noalloc: device memory the library holds itself.
// Each GPU the library runs on gets its own copy when the code object is loaded there, kept until
// the process ends. In host code `scratch` names a host-side stand-in, not device memory: only
// the per-device addresses from hipGetSymbolAddress are ever passed to kernels.
static __device__ __align__(256) char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up on the first call made with
// that device current and kept for later calls.
int scratch_of_current_device(const char* who, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return pa::set_error(PA_ERR_HIP, "%s: hipGetDevice: %s", who, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return pa::set_error(PA_ERR_HIP, "%s: device %d beyond the %d this library tracks", who, dev,
                         kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return pa::set_error(PA_ERR_HIP, "%s: hipGetSymbolAddress(scratch): %s", who,
                           hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" int paged_attn_varlen_prefill_noalloc(
    const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
    int32_t max_blocks_per_seq, const int32_t* cu_seqlens_q, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, float scale, int32_t dtype, const pa_task* tasks_dev,
    int32_t num_tasks, uint32_t task_kinds, const pa_combine* combines_dev,
    int32_t num_combines, int32_t num_partials, void* out, void* stream) {
  const char* who = "paged_attn_varlen_prefill_noalloc";
  if (int rc = varlen_checks(who, q, k_pages, v_pages, block_table, max_blocks_per_seq,
                             cu_seqlens_q, context_lens, num_seqs, num_tokens, num_q_heads,
                             num_kv_heads, head_dim, block_size, dtype, tasks_dev, num_tasks,
                             task_kinds, combines_dev, num_combines, num_partials, out))
    return rc;
  const bool partials = num_partials > 0 || num_combines > 0;
  if (partials) {
    const size_t need = pa_workspace_bytes(num_partials, head_dim);
    if (need > PA_NOALLOC_SCRATCH_BYTES)
      return pa::set_error(PA_ERR_CAPACITY,
                           "%s: %d partial rows need %zu bytes; this entry holds %zu (use "
                           "paged_attn_varlen_prefill with a workspace)",
                           who, num_partials, need, static_cast<size_t>(PA_NOALLOC_SCRATCH_BYTES));
  }
  if (num_tasks == 0) return pa::clear_error();
  // every partial row the combine reads is written by a task of the same launch before it, so
  // nothing in the scratch has to start at zero
  void* ws = nullptr;
  if (partials)
    if (int rc = scratch_of_current_device(who, &ws)) return rc;
  return varlen_enqueue(who, q, k_pages, v_pages, block_table, max_blocks_per_seq, cu_seqlens_q,
                        context_lens, num_q_heads, num_kv_heads, head_dim, block_size, scale,
                        tasks_dev, num_tasks, combines_dev, num_combines, num_partials,
                        task_kinds, ws, out, stream);
}

extern "C" int reshape_and_cache_fp8(const void* k_new, const void* v_new, void* k_pages,
                                     void* v_pages, float* scales,
                                     const int32_t* block_table, int32_t max_blocks_per_seq,
                                     const int32_t* cu_seqlens_q, const int32_t* context_lens,
                                     int32_t num_seqs, int32_t num_tokens, int32_t num_blocks,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                     void* stream) {
  if (num_tokens < 0 || num_seqs < 0 || num_blocks < 0 || max_blocks_per_seq < 0)
    return pa::set_error(PA_ERR_SHAPE, "reshape_and_cache_fp8: negative size");
  if (num_tokens > pa::kMaxWorkgroups)
    return pa::set_error(PA_ERR_SHAPE,
                         "reshape_and_cache_fp8: %d tokens: one launch takes at most %d",
                         num_tokens, pa::kMaxWorkgroups);
  if (num_kv_heads < 1 || !pa::head_dim_ok(head_dim))
    return pa::set_error(PA_ERR_SHAPE, "reshape_and_cache_fp8: Hkv %d, head_dim %d", num_kv_heads,
                         head_dim);
  if (!pa::block_size_ok(block_size))
    return pa::set_error(PA_ERR_BLOCK_SIZE, "reshape_and_cache_fp8: block_size %d", block_size);
  if (num_tokens == 0) return pa::clear_error();
  if (!k_new || !v_new || !k_pages || !v_pages || !scales || !block_table || !cu_seqlens_q ||
      !context_lens)
    return pa::set_error(PA_ERR_NULL, "reshape_and_cache_fp8: NULL pointer");
  if (num_seqs < 1)
    return pa::set_error(PA_ERR_SHAPE, "reshape_and_cache_fp8: tokens without sequences");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int shift = log2i(block_size);
  const unsigned units = (2 * num_kv_heads + kThreads / 64 - 1) / (kThreads / 64);
  // runs of tokens per workgroup: one token each up to kFp8WriteRuns tokens (decode batches:
  // every token starts its page), longer runs beyond (prefill chunks: one page per block)
  constexpr int kFp8WriteRuns = 4096;
  const int per_group = (num_tokens + kFp8WriteRuns - 1) / kFp8WriteRuns;
  const int groups = (num_tokens + per_group - 1) / per_group;
#define PA_RC8_LAUNCH(DD)                                                                      \
  hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<DD>, dim3(groups, units), dim3(kThreads), 0, st, \
                     static_cast<const __bf16*>(k_new), static_cast<const __bf16*>(v_new),      \
                     static_cast<uint8_t*>(k_pages), static_cast<uint8_t*>(v_pages), scales,    \
                     block_table, max_blocks_per_seq, cu_seqlens_q, context_lens,               \
                     num_seqs, num_tokens, per_group, num_kv_heads, block_size, shift)
  if (head_dim == 128)
    PA_RC8_LAUNCH(128);
  else
    PA_RC8_LAUNCH(64);
#undef PA_RC8_LAUNCH
  return hip_check("reshape_and_cache_fp8");
}

extern "C" int paged_attn_decode_fp8(const void* q, const void* k_pages, const void* v_pages,
                                     const float* scales,
                                     const int32_t* block_table, int32_t max_blocks_per_seq,
                                     const int32_t* context_lens, int32_t num_seqs,
                                     int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t block_size, float scale,
                                     const pa_task* tasks_dev, int32_t num_tasks,
                                     uint32_t task_kinds, const pa_combine* combines_dev,
                                     int32_t num_combines, int32_t num_partials,
                                     void* workspace, size_t workspace_bytes, void* out,
                                     void* stream) {
  if (int rc = check_attn_scalars("paged_attn_decode_fp8", num_seqs, num_q_heads, num_kv_heads,
                                  head_dim, block_size, PA_BF16, num_tasks, num_combines,
                                  num_partials, workspace_bytes, workspace, max_blocks_per_seq))
    return rc;
  if (int rc = check_kinds("paged_attn_decode_fp8", num_tasks, task_kinds, kDecodeKinds))
    return rc;
  if (num_tasks == 0) return pa::clear_error();
  if (!q || !k_pages || !v_pages || !scales || !block_table || !context_lens || !out ||
      !tasks_dev || (num_combines > 0 && !combines_dev))
    return pa::set_error(PA_ERR_NULL, "paged_attn_decode_fp8: NULL pointer");
  hipStream_t st = static_cast<hipStream_t>(stream);
  AttnArgs a = make_args(q, k_pages, v_pages, block_table, max_blocks_per_seq, nullptr,
                         context_lens, num_q_heads, num_kv_heads, head_dim, block_size, scale,
                         tasks_dev, num_tasks, num_partials, workspace, out);
  a.scales = scales;
  if (head_dim == 128) {
    hipLaunchKernelGGL(decode_fp8_kernel<128>, dim3(num_tasks), dim3(kThreads), 0, st, a);
    launch_combine<__bf16, 128>(combines_dev, num_combines, nullptr, a, st);
  } else {
    hipLaunchKernelGGL(decode_fp8_kernel<64>, dim3(num_tasks), dim3(kThreads), 0, st, a);
    launch_combine<__bf16, 64>(combines_dev, num_combines, nullptr, a, st);
  }
  return hip_check("paged_attn_decode_fp8");
}

extern "C" int paged_attn_verify_fp8(const void* q, const void* k_pages, const void* v_pages,
                                     const float* scales,
                                     const int32_t* block_table, int32_t max_blocks_per_seq,
                                     const int32_t* cu_seqlens_q, const int32_t* context_lens,
                                     int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                     float scale, const pa_task* tasks_dev, int32_t num_tasks,
                                     uint32_t task_kinds, const pa_combine* combines_dev,
                                     int32_t num_combines, int32_t num_partials,
                                     void* workspace, size_t workspace_bytes, void* out,
                                     void* stream) {
  if (int rc = check_attn_scalars("paged_attn_verify_fp8", num_seqs, num_q_heads, num_kv_heads,
                                  head_dim, block_size, PA_BF16, num_tasks, num_combines,
                                  num_partials, workspace_bytes, workspace, max_blocks_per_seq))
    return rc;
  if (int rc = check_kinds("paged_attn_verify_fp8", num_tasks, task_kinds, kVerifyKinds))
    return rc;
  if (num_tokens < num_seqs)
    return pa::set_error(PA_ERR_SHAPE, "paged_attn_verify_fp8: %d tokens for %d sequences",
                         num_tokens, num_seqs);
  if (num_tasks == 0) return pa::clear_error();
  if (!q || !k_pages || !v_pages || !scales || !block_table || !cu_seqlens_q || !context_lens ||
      !out || !tasks_dev || (num_combines > 0 && !combines_dev))
    return pa::set_error(PA_ERR_NULL, "paged_attn_verify_fp8: NULL pointer");
  hipStream_t st = static_cast<hipStream_t>(stream);
  AttnArgs a = make_args(q, k_pages, v_pages, block_table, max_blocks_per_seq, cu_seqlens_q,
                         context_lens, num_q_heads, num_kv_heads, head_dim, block_size, scale,
                         tasks_dev, num_tasks, num_partials, workspace, out);
  a.scales = scales;
  if (head_dim == 128) {
    hipLaunchKernelGGL(decode_fp8_kernel<128>, dim3(num_tasks), dim3(kThreads), 0, st, a);
    launch_combine<__bf16, 128>(combines_dev, num_combines, cu_seqlens_q, a, st);
  } else {
    hipLaunchKernelGGL(decode_fp8_kernel<64>, dim3(num_tasks), dim3(kThreads), 0, st, a);
    launch_combine<__bf16, 64>(combines_dev, num_combines, cu_seqlens_q, a, st);
  }
  return hip_check("paged_attn_verify_fp8");
}

extern "C" int paged_attn_varlen_prefill_fp8(
    const void* q, const void* k_pages, const void* v_pages, const float* scales,
    const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* cu_seqlens_q,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
    const pa_task* tasks_dev, int32_t num_tasks, uint32_t task_kinds,
    const pa_combine* combines_dev, int32_t num_combines, int32_t num_partials, void* workspace,
    size_t workspace_bytes, void* out, void* stream) {
  const char* who = "paged_attn_varlen_prefill_fp8";
  if (int rc = varlen_checks(who, q, k_pages, v_pages, block_table, max_blocks_per_seq,
                             cu_seqlens_q, context_lens, num_seqs, num_tokens, num_q_heads,
                             num_kv_heads, head_dim, block_size, PA_BF16, tasks_dev, num_tasks,
                             task_kinds, combines_dev, num_combines, num_partials, out))
    return rc;
  if (int rc = check_workspace(who, num_partials, num_combines, head_dim, workspace_bytes,
                               workspace))
    return rc;
  if (num_tasks == 0) return pa::clear_error();
  if (!scales) return pa::set_error(PA_ERR_NULL, "%s: NULL pointer", who);
  return varlen_enqueue(who, q, k_pages, v_pages, block_table, max_blocks_per_seq, cu_seqlens_q,
                        context_lens, num_q_heads, num_kv_heads, head_dim, block_size, scale,
                        tasks_dev, num_tasks, combines_dev, num_combines, num_partials,
                        task_kinds, workspace, out, stream, scales);
}
