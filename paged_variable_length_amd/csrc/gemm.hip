// SmoothGEMM for gfx950: C = A W^T for arbitrary M, N, K in fixed square tiles, driven by a
// load-sorted task table (XY-Serve page, section 2.2 "SmoothGEMM", and section 4.4,
// decompose_linear).
//
// Virtual padding (XY-Serve page, section 2.2): nothing is padded in memory. A tile at the edge
// of the output loads only the rows that exist -- the loads of missing rows are switched off
// lane by lane, so those LDS rows keep whatever they held, which reaches only output rows and
// columns that are never stored -- and the reduction tail past the task's K range is written
// into LDS as zeros, so it adds nothing to the valid outputs. Stores write valid elements only.
//
// Layouts: A [M, K], W [N, K] (a Linear layer's weight; both operands contiguous along K),
// C [M, N], all bf16 row-major; fp32 accumulation; C rounded to nearest even.
//
// One workgroup per task. The task's output tile (TILE x TILE) is split between the waves
// (2 x 4 waves of 128 x 64 for TILE 256, 2 x 2 waves of 64 x 64 for TILE 128, so the
// accumulators fit two waves per SIMD); each wave computes 32 x 32 blocks of C^T on 32x32x16
// bf16 MFMAs with a W block as the A operand and an A block as the B operand, so a lane holds
// one row of C and runs of four consecutive columns (8-byte stores). The reduction runs in stages of 64: A and W
// tiles [TILE rows][64] go through LDS, two buffers each, written by direct global->LDS loads
// (16 bytes per lane). Rows are 128 bytes (8 chunks of 16); logical chunk c of row r sits at
// position c ^ ((r >> 1) & 7), so the 16 lanes that read one chunk of 16 consecutive rows hit
// 16 distinct bank groups. The permutation is applied on the global side of the direct load
// (each 128-byte row segment is still read whole by 8 lanes).
//
// Pipeline: the k-steps (16 deep, four per stage) run as one sequence; the operands of k-step
// u+1 are read from LDS into one register set while the MFMAs of k-step u use the other.
// Before the last k-step of stage s each wave waits for its share of stage s+1's loads, and a
// barrier makes every share visible and marks stage s's buffers as read by all waves; right
// after it the loads of stage s+2 go into those buffers, so each load has about 1.75 stages of
// matrix work to land.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kReduceThreads = 256;
// Largest table run with the four-stage ring: one task per CU of the chip (256 CUs).
constexpr int kDeepRingMaxTasks = 256;

// Wave grid of a tile: WAVES_M x WAVES_N waves, each owning (TILE / WAVES_M) rows and
// (TILE / WAVES_N) columns of the output tile.
template <int TILE>
struct GemmCfg {
  static constexpr int kWavesM = 2;
  static constexpr int kWavesN = TILE == 256 ? 4 : 2;
  static constexpr int kWaves = kWavesM * kWavesN;
  static constexpr int kThreads = 64 * kWaves;
};
constexpr int kBK = 64;             // reduction depth of one stage
constexpr int kRowBytes = kBK * 2;  // one bf16 row of a stage tile

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return static_cast<uint16_t>(pack_bf16x2(x, 0.f) & 0xffffu);
}

// Position of logical chunk c in tile row r (a permutation of the row's 8 chunks, its own
// inverse).
__device__ __forceinline__ int chunk_pos(int r, int c) { return c ^ ((r >> 1) & 7); }

struct GemmArgs {
  const uint16_t* a;
  const uint16_t* w;
  uint16_t* c;
  float* ws;                   // partial tiles [num_slots][TILE][TILE] fp32
  const pa_gemm_task* tasks;
  int32_t M, N, K;
  int32_t num_tasks;
};

// Workgroups are dispatched round-robin over the 8 XCDs. Inside each full window of 64
// consecutive workgroups, XCD x takes table entries 8x .. 8x+7: with equal loads these are
// neighbouring column blocks of one row block (emission order), whose A rows then meet in one
// L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int base = bid & ~63;
  if (base + 64 > n) return bid;
  const int r = bid & 63;
  return base + (r & 7) * 8 + (r >> 3);
}

// N reads of 16 bytes at lane addresses a[i] + OFF (asm: the compiler cannot tell that these
// never touch the buffers the direct loads are filling and would wait for those loads first).
// Results are valid only after lds_wait.
template <int OFF, int N>
__device__ __forceinline__ void lds_read_n(const uint32_t (&a)[N], u32x4 (&r)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i)
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=&v"(r[i]) : "v"(a[i]), "n"(OFF) : "memory");
}

// Waits until at most K LDS operations are outstanding, tied to the registers of r: LDS
// operations complete in issue order, so with K = the number issued after r's reads, r holds
// its data afterwards (older extra operations only make the wait stronger).
template <int K, int N>
__device__ __forceinline__ void lds_wait(u32x4 (&r)[N]) {
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(K) : "memory");
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(r[i]));
}

// Waits until at most N of this wave's vector memory operations are outstanding (N < 64).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // vmcnt bits 3:0 and 15:14; expcnt (6:4) and lgkmcnt (11:8) at their maxima: no wait on them
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// TILE x TILE output tile per workgroup (128 or 256). ALIGNED: K % 8 == 0 and 16-byte aligned
// bases, so every 16-byte chunk of a row is whole and aligned and stages load through direct
// global->LDS loads; otherwise each lane gathers its chunk element by element into registers and
// writes it (same layout, slower). NS: stage buffers per operand. With NS = 2 a stage's loads
// are issued one stage ahead of its use; with NS = 4 (tile 128 only: 128 KiB of LDS, one
// workgroup per CU, for tables with at most one task per CU) three stages ahead, so a stage of
// small products no longer waits out the whole memory latency.
template <int TILE, bool ALIGNED, int NS>
__global__ __launch_bounds__(GemmCfg<TILE>::kThreads) void smooth_gemm_kernel(GemmArgs g) {
  static_assert(NS == 2 || (NS == 4 && TILE == 128 && ALIGNED), "four stages: aligned tile 128");
  typedef GemmCfg<TILE> C;
  constexpr int WM = TILE / C::kWavesM;             // wave tile rows (m)
  constexpr int WN = TILE / C::kWavesN;             // wave tile columns (n)
  constexpr int NBM = WM / 32, NBN = WN / 32;       // 32-wide MFMA blocks per wave tile
  constexpr int kTileBytes = TILE * kRowBytes;      // one operand, one stage
  constexpr int kPieces = kTileBytes / 1024 / C::kWaves;   // 1 KiB loads per wave per operand
  static_assert(kPieces % 2 == 0, "pieces per wave must be even");
  constexpr int NOPS = NBN + NBM;                   // operand registers per k-step
  __shared__ __attribute__((aligned(1024))) char smem[2 * NS * kTileBytes];   // A0.. W0..

  const pa_gemm_task t = g.tasks[xcd_remap(blockIdx.x, g.num_tasks)];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / C::kWavesN, wn = wave % C::kWavesN;
  const int m0 = __builtin_amdgcn_readfirstlane(t.m0);
  const int rows = __builtin_amdgcn_readfirstlane(t.rows);
  const int n0 = __builtin_amdgcn_readfirstlane(t.n0);
  const int cols = __builtin_amdgcn_readfirstlane(t.cols);
  const int k0 = __builtin_amdgcn_readfirstlane(t.k0);
  const int k1 = __builtin_amdgcn_readfirstlane(t.k1);
  const int slot = __builtin_amdgcn_readfirstlane(t.slot);
  const int K = g.K;
  const int nst = (k1 - k0 + kBK - 1) / kBK;

  // ---- loads of stage s into buffer `buf`: piece q of this wave covers tile rows
  // 8*(wave*kPieces + q) .. +7; lane L takes row +L/8 at position L%8, i.e. the logical chunk
  // chunk_pos(row, L%8). wave*kPieces is even, so that chunk depends on q only through q & 1:
  // lane offsets (element units, relative to the piece's first row) for even and odd pieces.
  const int lrow = lane >> 3, lpos = lane & 7;
  int loff[2] = {lrow * K + 8 * chunk_pos(lrow, lpos), lrow * K + 8 * chunk_pos(8 + lrow, lpos)};
  int lchunk[2] = {8 * chunk_pos(lrow, lpos), 8 * chunk_pos(8 + lrow, lpos)};
  auto load_stage = [&](int s, int buf) {
    const int ks = k0 + s * kBK;
    // opaque redefinition: the lane offsets are not folded into per-piece addresses held
    // across the loop
    asm volatile("" : "+v"(loff[0]), "+v"(loff[1]), "+v"(lchunk[0]), "+v"(lchunk[1]));
#pragma unroll
    for (int op = 0; op < 2; ++op) {
      const uint16_t* src = op == 0 ? g.a : g.w;
      const int base_row = op == 0 ? m0 : n0;
      const int nrows = op == 0 ? rows : cols;
      char* tile = smem + (NS * op + buf) * kTileBytes;
      // every row of the tile exists and the stage is a whole 64: no lane is switched off
      const bool interior = nrows == TILE && ks + kBK <= k1;
      if constexpr (ALIGNED && C::kWaves == 8) {
        if (interior) {
          // waves 0-3 load the pieces of waves w and w+4 and waves 4-7 load nothing: waves w
          // and w+4 share a SIMD, so one of them can wait on its loads while the other keeps
          // the matrix pipe busy (measured: +8% over every wave loading its own pieces, and
          // better than alternating the loading half by stage)
          if (wave < 4) {
#pragma unroll
            for (int half = 0; half < 2; ++half)
#pragma unroll
              for (int q = 0; q < kPieces; ++q) {
                const int slot = (wave + 4 * half) * kPieces + q;
                const uint16_t* piece = src + static_cast<size_t>(base_row + 8 * slot) * K + ks;
                __builtin_amdgcn_global_load_lds(
                    piece + loff[q & 1],
                    (__attribute__((address_space(3))) void*)(tile + slot * 1024), 16, 0, 0);
              }
          }
          continue;
        }
      }
#pragma unroll
      for (int q = 0; q < kPieces; ++q) {
        const int r0 = 8 * (wave * kPieces + q);          // the piece's first tile row
        const int kc = ks + lchunk[q & 1];
        char* dst = tile + (wave * kPieces + q) * 1024;
        const bool row_ok = r0 + lrow < nrows;
        if constexpr (ALIGNED) {
          const uint16_t* piece = src + static_cast<size_t>(base_row + r0) * K + ks;
          if (interior) {
            __builtin_amdgcn_global_load_lds(piece + loff[q & 1],
                                             (__attribute__((address_space(3))) void*)dst, 16,
                                             0, 0);
            continue;
          }
          // K % 8 == 0 and k1 is K or a multiple of 64: a chunk lies wholly inside [k0, k1)
          // or wholly past it
          if (kc >= k1) {
            *reinterpret_cast<u32x4*>(dst + lane * 16) = u32x4{0u, 0u, 0u, 0u};
          } else if (row_ok) {
            __builtin_amdgcn_global_load_lds(piece + loff[q & 1],
                                             (__attribute__((address_space(3))) void*)dst, 16,
                                             0, 0);
          }
        } else {
          const uint16_t* row = src + static_cast<size_t>(base_row + r0 + lrow) * K;
          uint32_t e[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) e[i] = (row_ok && kc + i < k1) ? row[kc + i] : 0u;
          *reinterpret_cast<u32x4*>(dst + lane * 16) =
              u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                    e[6] | (e[7] << 16)};
        }
      }
    }
  };

  // ---- operand addresses. Lane (j = lane%32, h = lane/32) reads row 32*blk + j of its
  // wave's rows, logical chunk 2*kk + h. Row bases are multiples of 128 bytes and rows
  // W*w + 32*blk + j share (r >> 1) & 7 with j, so k-step kk is the k-step-0 address XOR
  // (kk << 5), and block blk and the buffer enter as offsets.
  const int j = lane & 31, h = lane >> 5;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem));
  uint32_t a_base = lds0 + (WM * wm + j) * kRowBytes + (chunk_pos(j, h) << 4);
  uint32_t w_base = lds0 + NS * kTileBytes + (WN * wn + j) * kRowBytes + (chunk_pos(j, h) << 4);

  // operands of one k-step: [0, NBN) W blocks (n), [NBN, NBN + NBM) A blocks (m)
  typedef u32x4 Ops[NOPS];
  auto read_ops = [&](uint32_t boff, int kk, Ops& o) {
    const uint32_t xo = static_cast<uint32_t>(kk) << 5;
    uint32_t ad[NOPS];
#pragma unroll
    for (int b = 0; b < NBN; ++b) ad[b] = (w_base ^ xo) + boff + b * 32 * kRowBytes;
#pragma unroll
    for (int b = 0; b < NBM; ++b) ad[NBN + b] = (a_base ^ xo) + boff + b * 32 * kRowBytes;
    lds_read_n<0>(ad, o);
  };

  f32x16 acc[NBN][NBM];   // [n block][m block] of C^T
#pragma unroll
  for (int x = 0; x < NBN; ++x)
#pragma unroll
    for (int y = 0; y < NBM; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.f;

  // MFMAs of n blocks [x0, x1) against every m block
  auto mfmas = [&](const Ops& o, int x0, int x1) {
#pragma unroll
    for (int x = 0; x < NBN; ++x) {
      if (x < x0 || x >= x1) continue;
#pragma unroll
      for (int y = 0; y < NBM; ++y)
        acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(o[x]), as_bf16x8(o[NBN + y]),
                                                           acc[x][y], 0, 0, 0);
    }
  };

  // Waits for this wave's loads of one stage while `after` later stages are in flight. A task
  // whose every stage is interior issues kLoads loads per wave per stage, so the wait counts
  // exactly; elsewhere lanes switch loads off at the edges and the wait is a full one.
  constexpr int kLoads = 2 * kPieces;
  const bool counted = NS > 2 && rows == TILE && cols == TILE && (k1 - k0) % kBK == 0;
  auto wait_stage = [&](int after) {
    if constexpr (NS > 2) {
      if (counted) {
        if (after == 3) {
          vm_wait<3 * kLoads>();
          return;
        }
        if (after == 2) {
          vm_wait<2 * kLoads>();
          return;
        }
        if (after == 1) {
          vm_wait<kLoads>();
          return;
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
  };

  // ---- prologue: stages 0 .. NS-1 in flight; wait for stage 0; operands of its first k-step
  for (int i = 0; i < NS; ++i)
    if (i < nst) load_stage(i, i);
  wait_stage(min(nst, NS) - 1);
  __builtin_amdgcn_s_barrier();
  Ops o0, o1;
  read_ops(0u, 0, o0);

  // ---- stage s (operands of its k-step 0 already requested into o0), buffer s % NS
  for (int s = 0; s < nst; ++s) {
    const uint32_t cur = static_cast<uint32_t>(s % NS) * kTileBytes;
    const uint32_t nxt = static_cast<uint32_t>((s + 1) % NS) * kTileBytes;
    // opaque redefinition: the per-k-step addresses are recomputed where used instead of being
    // held in registers across the loop
    asm volatile("" : "+v"(a_base), "+v"(w_base));
    read_ops(cur, 1, o1);
    lds_wait<NOPS>(o0);
    mfmas(o0, 0, NBN);
    read_ops(cur, 2, o0);
    lds_wait<NOPS>(o1);
    mfmas(o1, 0, NBN);
    read_ops(cur, 3, o1);
    lds_wait<NOPS>(o0);
    mfmas(o0, 0, NBN);
    // stage s+1's loads landed (this wave's share) and every wave's k-step-3 operands arrived;
    // after the barrier stage s's buffers are free. The scheduling fences keep the matrix
    // steps of k-step 2 ahead of the wait (the matrix pipe works while the wave waits) and
    // the loads of stage s+2 between the two halves of k-step 3.
    __builtin_amdgcn_sched_barrier(0);
    lds_wait<0>(o1);
    // stages s+2 .. min(nst, s+NS) - 1 were issued after stage s+1
    wait_stage(max(0, min(nst, s + NS) - s - 2));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    mfmas(o1, 0, NBN / 2);
    __builtin_amdgcn_sched_barrier(0);
    if (s + NS < nst) load_stage(s + NS, s % NS);
    if (s + 1 < nst) read_ops(nxt, 0, o0);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(o1, NBN / 2, NBN);
  }

  // ---- epilogue. Lane (j, h) holds, for m block y and n block x, row m = WM*wm + 32y + j and
  // columns n = WN*wn + 32x + 8*rb + 4h + (0..3) in acc[x][y][4rb .. 4rb+3] (tile-relative).
  if (slot < 0) {
    const bool vec = (g.N & 3) == 0 && (reinterpret_cast<uintptr_t>(g.c) & 7) == 0;
#pragma unroll
    for (int y = 0; y < NBM; ++y) {
      const int mr = WM * wm + 32 * y + j;
      if (mr >= rows) continue;
      uint16_t* crow = g.c + static_cast<size_t>(m0 + mr) * g.N + n0;
#pragma unroll
      for (int x = 0; x < NBN; ++x)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const int nc = WN * wn + 32 * x + 8 * rb + 4 * h;
          const f32x16& v = acc[x][y];
          if (vec && nc + 3 < cols) {
            *reinterpret_cast<u32x2*>(crow + nc) =
                u32x2{pack_bf16x2(v[4 * rb], v[4 * rb + 1]), pack_bf16x2(v[4 * rb + 2], v[4 * rb + 3])};
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (nc + e < cols) crow[nc + e] = bf16_bits(v[4 * rb + e]);
          }
        }
    }
  } else {
    // fp32 partial tile [TILE][TILE]; rows and columns past the valid region are never read
    float* pt = g.ws + static_cast<size_t>(slot) * TILE * TILE;
#pragma unroll
    for (int y = 0; y < NBM; ++y) {
      const int mr = WM * wm + 32 * y + j;
#pragma unroll
      for (int x = 0; x < NBN; ++x)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const int nc = WN * wn + 32 * x + 8 * rb + 4 * h;
          const f32x16& v = acc[x][y];
          *reinterpret_cast<f32x4*>(pt + mr * TILE + nc) =
              f32x4{v[4 * rb], v[4 * rb + 1], v[4 * rb + 2], v[4 * rb + 3]};
        }
    }
  }
}

// Sum of the fp32 partial tiles of one output block, rounded to bf16 into C (valid elements
// only). Workgroup b takes reduce record b / groups and rows (b % groups) * RPB .. + RPB - 1;
// thread t covers four consecutive columns.
template <int TILE>
__global__ __launch_bounds__(kReduceThreads) void gemm_reduce_kernel(const pa_gemm_reduce* reds,
                                                                   const float* ws, uint16_t* c,
                                                                   int32_t N) {
  constexpr int TPR = TILE / 4;             // threads per row
  constexpr int RPB = kReduceThreads / TPR;   // rows per workgroup
  constexpr int GROUPS = TILE / RPB;
  const pa_gemm_reduce rd = reds[blockIdx.x / GROUPS];
  const int r = (blockIdx.x % GROUPS) * RPB + threadIdx.x / TPR;
  const int cc = (threadIdx.x % TPR) * 4;
  if (r >= rd.rows || cc >= rd.cols) return;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < rd.n_slots; ++k)
    s += *reinterpret_cast<const f32x4*>(ws + static_cast<size_t>(rd.first_slot + k) * TILE * TILE +
                                         r * TILE + cc);
  uint16_t* crow = c + static_cast<size_t>(rd.m0 + r) * N + rd.n0;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (cc + e < rd.cols) crow[cc + e] = bf16_bits(s[e]);
}

template <int TILE>
int launch_gemm(const GemmArgs& g, bool aligned, const pa_gemm_reduce* reds, int32_t num_reduces,
                hipStream_t st) {
  if (g.num_tasks > 0) {
    // a tile-128 table of at most one task per CU runs with the deeper stage ring (one
    // workgroup per CU)
    if (TILE == 128 && aligned && g.num_tasks <= kDeepRingMaxTasks)
      hipLaunchKernelGGL((smooth_gemm_kernel<128, true, 4>), dim3(g.num_tasks),
                         dim3(GemmCfg<128>::kThreads), 0, st, g);
    else if (aligned)
      hipLaunchKernelGGL((smooth_gemm_kernel<TILE, true, 2>), dim3(g.num_tasks),
                         dim3(GemmCfg<TILE>::kThreads), 0, st, g);
    else
      hipLaunchKernelGGL((smooth_gemm_kernel<TILE, false, 2>), dim3(g.num_tasks),
                         dim3(GemmCfg<TILE>::kThreads), 0, st, g);
  }
  if (num_reduces > 0) {
    constexpr int GROUPS = TILE / (kReduceThreads / (TILE / 4));
    hipLaunchKernelGGL((gemm_reduce_kernel<TILE>), dim3(num_reduces * GROUPS), dim3(kReduceThreads),
                       0, st, reds, g.ws, g.c, g.N);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pa::set_error(PA_ERR_HIP, "smooth_gemm: launch failed: %s",
                                            hipGetErrorString(e));
  return pa::clear_error();
}

}  // namespace

extern "C" size_t pa_gemm_workspace_bytes(int32_t num_slots, int32_t tile) {
  if (num_slots <= 0 || (tile != 128 && tile != 256)) return 0;
  const size_t b = static_cast<size_t>(num_slots) * tile * tile * sizeof(float);
  return (b + 255) & ~static_cast<size_t>(255);
}

extern "C" int smooth_gemm(const void* a, const void* w, void* c, int32_t M, int32_t N, int32_t K,
                           int32_t tile, const pa_gemm_task* tasks_dev, int32_t num_tasks,
                           const pa_gemm_reduce* reduces_dev, int32_t num_reduces,
                           int32_t num_slots, void* workspace, size_t workspace_bytes,
                           void* stream) {
  if (M < 0 || N < 0 || K < 0 || num_tasks < 0 || num_reduces < 0 || num_slots < 0)
    return pa::set_error(PA_ERR_SHAPE, "smooth_gemm: negative size or count");
  if (tile != 128 && tile != 256)
    return pa::set_error(PA_ERR_SHAPE, "smooth_gemm: tile %d must be 128 or 256", tile);
  // the reduce launch runs tile^2 / (4 kReduceThreads) workgroups per record (each thread sums
  // four columns of one row)
  const int64_t reduce_groups =
      static_cast<int64_t>(num_reduces) * tile * tile / (4 * kReduceThreads);
  if (num_tasks > pa::kMaxWorkgroups || reduce_groups > pa::kMaxWorkgroups)
    return pa::set_error(PA_ERR_SHAPE, "smooth_gemm: %d tasks, %d reduces exceed one launch",
                         num_tasks, num_reduces);
  if (num_tasks == 0) return pa::clear_error();
  if (M == 0 || N == 0 || K == 0)
    return pa::set_error(PA_ERR_SHAPE, "smooth_gemm: tasks given for an empty product");
  if (!a || !w || !c || !tasks_dev || (num_reduces > 0 && !reduces_dev))
    return pa::set_error(PA_ERR_NULL, "smooth_gemm: NULL pointer");
  if (num_reduces > 0 && (!workspace || workspace_bytes < pa_gemm_workspace_bytes(num_slots, tile)))
    return pa::set_error(PA_ERR_CAPACITY, "smooth_gemm: workspace of %zu bytes, %zu needed",
                         workspace_bytes, pa_gemm_workspace_bytes(num_slots, tile));
  GemmArgs g;
  g.a = static_cast<const uint16_t*>(a);
  g.w = static_cast<const uint16_t*>(w);
  g.c = static_cast<uint16_t*>(c);
  g.ws = static_cast<float*>(workspace);
  g.tasks = tasks_dev;
  g.M = M;
  g.N = N;
  g.K = K;
  g.num_tasks = num_tasks;
  const bool aligned = (K % 8) == 0 && (reinterpret_cast<uintptr_t>(a) & 15) == 0 &&
                       (reinterpret_cast<uintptr_t>(w) & 15) == 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return tile == 256 ? launch_gemm<256>(g, aligned, reduces_dev, num_reduces, st)
                     : launch_gemm<128>(g, aligned, reduces_dev, num_reduces, st);
}
