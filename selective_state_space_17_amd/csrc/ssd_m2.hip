// Mamba-2 scalar-A multi-head ("SSD") forward for gfx950 (MI355X), with the
// Mamba-3 input rules on the same block form: the exponential-trapezoidal rule
// and several inputs and outputs per channel (MIMO).
//
// Per (batch b, head h, headdim p, state n) with group g = h / (H / G):
//   S[p,n] <- exp(delta_t A_h) S[p,n] + delta_t B[t,g,n] x[t,h,p]
//   y[t,h,p] = sum_n C[t,g,n] S[p,n] (+ D_h x) (* silu(z))
// The transition is a scalar times the identity ("Mamba-3" blog,
// introduction), so within a block of steps the recurrence unrolls into
// matrix products ("Mamba-2 y state-space models", 4.2: the selective SSM
// written as matmuls).  With l_t = delta_t A_h and the inclusive in-block sum
// s_t = sum_{r<=t} l_r:
//   y_t   = exp(s_t) C_t . S_in  +  sum_{s<=t} (C_t . B_s) exp(s_t - s_s) w_s x_s
//   S_out = exp(s_Q) S_in + sum_s exp(s_Q - s_s) w_s x_s (x) B_s
// with w_s = delta_s (Mamba-2 rule).
//
// Mamba-3 exponential-trapezoidal rule ("Mamba-3" blog, "El modelo Mamba-3"
// item 1): S_t = a_t S_{t-1} + (1 - lam_t) d_t a_t x_{t-1} B_{t-1} + lam_t d_t x_t B_t.
// x_s reaches step t > s through one decay exp(s_t - s_s) with the summed
// weight lam_s d_s + (1 - lam_{s+1}) d_{s+1}, and its own step with lam_s d_s:
// only the weights change, and the state leaving a block already holds the
// next block's left-end term.  At the end of the sequence that term does not
// exist, so final_state is the plain S_{L-1}.
//
// Mamba-3 MIMO (item 3: several SSMs per update on one state; "Arquitectura":
// B and C widened): channel p of a head takes R inputs x[t,h,r,p] and gives R
// outputs, all on the head's one state; B[t,g,r,:] carries input r and
// C[t,g,r,:] reads output r.  A head's sequence is then L*R rows, row i being
// step i / R and rank i % R; the rows of a step share its decay and weights.
// The block form above holds over rows with "s <= t" read on steps: the
// state update sums R outer products per step and C . B^T couples every
// rank pair.  R = 1 is the single-input form.
//
// Mapping onto the chip.  A block is 64 rows.  One workgroup of 8 waves owns
// one (b, head, 64-wide headdim slice) and walks its sequence; the waves take
// two roles, one of each on every SIMD, so that the two waves sharing a SIMD
// do different work at the same time:
//  * state waves 0-3: wave w holds headdim columns 16 w .. 16 w + 15 of the
//    transposed state S^T[n, p] for all states, in MFMA accumulators for the
//    whole sequence (the state never leaves the chip except as final_state);
//    they read out the carried state, update it, and finish the outputs;
//  * mask waves 4-7: wave 4 + t forms the mask tiles of row tile t and the
//    per-row arrays (decay sums and weights) of the next block.
// Per block (v_mfma_f32_16x16x32_bf16, base-2 exponents, A pre-scaled by log2 e):
//   G^T = B . C^T   (s x t) all 16 tiles, tiles past the diagonal come out 0
//   M   = G o exp2(s_t - s_s) o w_s  ->  LDS as bf16 hi/lo, double-buffered
//   Y^T = exp2(s_t) (S . C^T) + X^T . M^T   (p x t)
//   S^T = exp2(s_Q) S^T + B^T . Xw          (n x p, k = rows)
// The X^T . M^T term of a block, with D x, the gate and the store, is done in
// the next block's pass of the state waves, once the barrier that starts it
// has published the mask: one barrier per block.  x, B and C enter the matrix
// cores exactly (bf16 inputs).  The three computed operands -- the state, the
// mask and the weighted inputs -- are each split into hi = bf16(v),
// lo = bf16(v - hi), about 16 significant bits: with one bf16 rounding the
// outputs drift past a 2e-2 relative bound in rare elements (the mask enters
// sums whose terms are much larger than the result).
//
// Data movement.  Every input reaches LDS by direct global->LDS loads
// (global_load_lds), shared out over all eight waves (a wave whose load finds
// the memory pipeline full waits, so one wave issuing them all would stall):
// x two blocks ahead, B and C one block ahead, delta and lam three blocks
// ahead.  Each tile in LDS is a plane of 64 rows x 128 bytes with row r's
// 16-byte chunk c kept at chunk c ^ (r % 8): 16-byte reads of one chunk from
// 16 consecutive rows and transposing reads of 8 consecutive rows are then both
// free of bank conflicts (B and C, 256-byte rows at 128 states, are split into
// two planes).  Fragments whose contraction index is the row index (B^T for
// the state update, X^T for the intra-block product) come from transposing LDS
// reads (ds_read_b64_tr_b16): in each 16-lane group, lane j receives element j
// of each of the four 4-element pieces that lanes 4k..4k+3 point at.  The
// state's readout fragments are brought into natural k order by two cross-lane
// swaps (v_permlane32_swap, v_permlane16_swap), so C is read 16 bytes at a
// time; the mask is stored in the k order of the X^T fragments for the same
// reason.  Each wave waits for its own loads (s_waitcnt vmcnt) and a barrier
// makes them visible; the loops hold no other vector-memory operations than
// these loads and the output stores, so the counts are exact and nothing
// drains the prefetch.  Within a pass, each phase issues all of its LDS reads
// before their first use.
#include <type_traits>

#include "internal.h"

namespace mssm {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kWave = 64;
constexpr int QB = 64;          // rows per block
constexpr int PB = 64;          // headdim slice per unit
constexpr int NXS = 3;          // x / z ring: two blocks ahead
constexpr int NBS = 2;          // B / C ring: one block ahead
constexpr int NDS = 4;          // delta / lam ring: three blocks ahead
// per-row arrays of a block (per unit): inclusive decay sum, exp2 of it, the
// weight at later steps, the weight at its own step, and the state-update weight
constexpr int A_CS = 0, A_ECS = 1, A_WF = 2, A_WD = 3, A_WL = 4, NARR = 5;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ float exp2_hw(float v) { return __builtin_amdgcn_exp2f(v); }
// two floats -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 8 floats -> bf16 hi/lo fragments (v = hi + lo to about 16 significant bits)
__device__ __forceinline__ void split8(const float (&v)[8], bf16x8& hi, bf16x8& lo) {
  u32x4 h, l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = pack2(v[2 * i], v[2 * i + 1]);
    l[i] = pack2(v[2 * i] - lo_f(h[i]), v[2 * i + 1] - hi_f(h[i]));
  }
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <typename T> __device__ __forceinline__ T lds_ld(const unsigned char* base, int byte) {
  return *reinterpret_cast<const T*>(base + byte);
}
// 8 bytes of a transposed read (see the header): returns 4 bf16
__device__ __forceinline__ u32x2 lds_tr(const unsigned char* base, int byte) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(const_cast<unsigned char*>(base) + byte));
  return __builtin_bit_cast(u32x2, v);
}
__device__ __forceinline__ bf16x8 cat(const u32x2 a, const u32x2 b) {
  return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
}

// global -> LDS: lane l's 16 bytes land at LDS offset lds + 16 l; a 2-byte load lands zero-extended in the
// dword at lds + 4 l.  lds is wave-uniform (it goes to M0); it is formed as an integer from each array's
// base, since a pointer chosen at run time among LDS buffers would be cast with a null check.  Written as asm so that the
// compiler does not track these loads: it would otherwise wait for all of them before the transposing
// LDS reads of the same buffers, draining the prefetch; completion is waited for explicitly (wait_vm)
// before the barrier that publishes a block.  The asm has no outputs (the data goes to LDS), so no
// register can be overwritten while a load is in flight.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  // the low half of a flat address into LDS is the LDS offset
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
__device__ __forceinline__ void dma2(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_ushort %0, off"
               :: "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}

// Barrier without a memory fence: LDS writes of this wave are complete
// first (lgkmcnt), direct loads were waited for by vmcnt before it.  The empty
// asm statements keep the compiler from moving LDS accesses across.
__device__ __forceinline__ void block_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// wait until at most n (0..8, wave-uniform) of this wave's vector-memory operations are outstanding.  Loads
// and stores share the counter and retire in issue order, so n counts the stores issued after the load
// waited for as well.
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
    case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}

// DPP-moved copy of v (lanes outside the row mask, or whose source lane is out
// of range, read 0)
template <int CTRL, int ROW_MASK> __device__ __forceinline__ float dppf(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf, true));
}

struct SSDParams {
  const uint16_t* x;
  const uint16_t* delta;
  const uint16_t* lam;   // exponential-trapezoidal weights [B, L, H] (TRAP only)
  const float* A;
  const uint16_t* B;
  const uint16_t* C;
  const float* D;
  const uint16_t* z;
  const float* h0;
  uint16_t* out;
  float* final_state;
  int64_t batch, L, H, P, N, G;
  int R, rs;     // inputs per channel (MIMO rank) and log2 R
  int nps;       // headdim slices per head (P / 64, rounded up; the last one is cut at P)
  // states n0 .. n0 + N - 1 of rows of Nr states (B, C, h0, final_state); with part != nullptr the
  // kernel writes this share of sum_n C S (+ the in-block term) in fp32 to part, [B, L, H, R, P], and
  // leaves D x, the gate and out to the kernel that adds the shares
  int64_t Nr, n0;
  float* part;
};

constexpr int kWaves = 8;
constexpr int kThreads = kWave * kWaves;
constexpr int PROW = 128;                // bytes of an LDS tile row: 64 bf16
constexpr int PLANE = QB * PROW;         // one 64-row tile (8 KB)

// Every tile in LDS is a plane of 64 rows x 128 bytes whose row r keeps its 16-byte chunk c at chunk
// c ^ (r % 8).  Both access shapes used below are then free of bank conflicts: 16-byte reads of one chunk
// from 16 consecutive rows, and transposing reads of 8 consecutive rows.
__device__ __forceinline__ int swz(int r, int c) { return r * PROW + ((c ^ (r & 7)) << 4); }

// What a state wave keeps from the main pass of a block for its finish in the next one: the carried-state
// readout of the four row tiles, the X^T fragments, and x (z) at the output points.
struct Carry {
  f32x4 y[4];
  bf16x8 xf0, xf1;
  u32x2 xv[4], zv[4];
};

// MFMA 16x16x32 lane layout: A row / B column = lane % 16, k slots 8(lane/16)..+7;
// accumulator element v of a lane is row 4 (lane / 16) + v, column lane % 16.
template <int NP, bool TRAP, bool EPI, bool PART>
__global__ __launch_bounds__(kThreads) void ssd_kernel(SSDParams p) {
  static_assert(NP == 64 || NP == 128, "padded state count");
  static_assert(!(EPI && PART), "a share of the states leaves D x and the gate to the kernel adding the shares");
  constexpr int NT = NP / 16;               // 16-row state tiles of a state wave
  constexpr int NKB = NP / 32;              // 32-wide k blocks over the states
  constexpr int NPL = NP / 64;              // planes of a B or C block
  constexpr int BBLK = NPL * PLANE;
  constexpr int NBC = 2 * NPL * 8;          // 1 KB loads of a block's B and C (8 rows of one plane each)
  constexpr int BC_PER = NBC / 8;           // per wave
  static_assert(NBC % 8 == 0, "B/C loads split evenly over the waves");

  __shared__ __attribute__((aligned(16))) unsigned char xs[NXS][PLANE];
  __shared__ __attribute__((aligned(16))) unsigned char zs[EPI ? NXS : 1][EPI ? PLANE : 16];
  __shared__ __attribute__((aligned(16))) unsigned char bs[NBS][BBLK];
  __shared__ __attribute__((aligned(16))) unsigned char cs_[NBS][BBLK];
  __shared__ __attribute__((aligned(16))) uint32_t dls[NDS][QB];            // delta bits, one per row
  __shared__ __attribute__((aligned(16))) uint32_t lls[TRAP ? NDS : 1][QB];   // lam bits
  __shared__ __attribute__((aligned(16))) unsigned char ms[2][2][PLANE];     // mask of even / odd blocks: hi, lo
  __shared__ __attribute__((aligned(16))) float arr[2][NARR][QB];
  static_assert(sizeof(xs) + sizeof(zs) + sizeof(bs) + sizeof(cs_) + sizeof(dls) + sizeof(lls) + sizeof(ms) +
                    sizeof(arr) <= 160 * 1024,
                "LDS budget");

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform, in a scalar register
  const bool state_wave = w < 4;       // waves 0-3 hold the state; waves 4-7 form the mask and the arrays
  const int pt = w & 3;                // state wave: 16-wide headdim tile; mask wave: 16-row t tile
  const int lc = lane % 16;
  const int q = lane / 16;

  // workgroup -> (b, g, head, slice); consecutive workgroups take different (b, g), so the heads of one
  // (b, g) share an XCD (and its L2, where B and C stay) when batch * groups is a multiple of 8
  const int64_t BG = p.batch * p.G;
  const int64_t bg = blockIdx.x % BG;
  const int64_t member = blockIdx.x / BG;
  const int64_t b = bg / p.G, g = bg % p.G;
  const int64_t hpg = p.H / p.G;
  const int64_t h = g * hpg + member / p.nps;
  const int64_t p0 = (member % p.nps) * PB;
  const int ncol = static_cast<int>(p.P - p0 < PB ? p.P - p0 : PB);   // columns of this slice (a multiple of 8)
  const int64_t L = p.L, H = p.H, P = p.P, N = p.N, G = p.G;
  const int R = p.R, rs = p.rs;
  const int Ni = static_cast<int>(N);
  const int spb = QB >> rs;            // steps per block
  const float a2 = p.A[h] * kLog2e;
  const float Dh = p.D != nullptr ? p.D[h] : 0.f;
  const bool has_z = p.z != nullptr;
  const int64_t nblocks = (L * R + QB - 1) / QB;
  const int last_nv = static_cast<int>(L * R - (nblocks - 1) * QB);   // rows of the last block

  // ---- zero what a load may leave untouched: B/C columns past N, and whatever an earlier kernel left ----
  {
    unsigned char* regions[5] = {&xs[0][0], &zs[0][0], &bs[0][0], &cs_[0][0], &ms[0][0][0]};
    const int sizes[5] = {static_cast<int>(sizeof(xs)), static_cast<int>(sizeof(zs)), static_cast<int>(sizeof(bs)),
                          static_cast<int>(sizeof(cs_)), static_cast<int>(sizeof(ms))};
#pragma unroll
    for (int r = 0; r < 5; ++r)
      for (int e = tid * 16; e < sizes[r]; e += kThreads * 16)
        *reinterpret_cast<u32x4*>(regions[r] + e) = u32x4{0, 0, 0, 0};
  }

  const int64_t Nr = p.Nr;   // B / C row length (all states)
  const int64_t xstep = H * R * P, bcstep = G * R * Nr;
  const uint16_t* const x0 = p.x + (b * L * H + h) * R * P + p0;         // step 0, rank 0 of this unit
  const uint16_t* const z0 = (has_z ? p.z : p.x) + (b * L * H + h) * R * P + p0;
  const uint16_t* const B0 = p.B + (b * L * G + g) * R * Nr + p.n0;
  const uint16_t* const C0 = p.C + (b * L * G + g) * R * Nr + p.n0;
  const uint16_t* const d0 = p.delta + b * L * H + h;
  const uint16_t* const l0 = TRAP ? p.lam + b * L * H + h : nullptr;
  uint16_t* const o0 = PART ? nullptr : p.out + (b * L * H + h) * R * P + p0;
  float* const po0 = PART ? p.part + (b * L * H + h) * R * P + p0 : nullptr;
  const uint32_t xs_a = lds_addr(&xs[0][0]), zs_a = lds_addr(&zs[0][0]), bs_a = lds_addr(&bs[0][0]),
                 cs_a = lds_addr(&cs_[0][0]), dls_a = lds_addr(&dls[0][0]), lls_a = lds_addr(&lls[0][0]);

  // ring slots, advanced by counters (no division in the loop)
  int sx = 0, sb = 0, sd = 0;   // slots of block k in the x, B/C and delta rings
  auto nxt = [](int v, int n) { return v + 1 == n ? 0 : v + 1; };
  auto advance = [&]() {
    sx = nxt(sx, NXS);
    sb = nxt(sb, NBS);
    sd = nxt(sd, NDS);
  };

  // ---- direct loads, shared out over all eight waves: wave w loads x (z) rows 8 w .. 8 w + 7, and B/C loads
  // BC_PER w .. +BC_PER-1 (8 rows of one plane each); waves 4 and 5 load delta and lam ----
  // a lane's row within its 8-row group and its logical 16-byte chunk (stored at chunk lane % 8 of the row);
  // a block's offsets are formed at issue time, rows past the block's valid ones clamped to its last
  const int lrow = lane / 8;
  // (cols: the row's valid columns; a chunk past them loads chunk 0 again, so every lane still loads)
  auto blk_off = [&](int64_t k, int row, int64_t step, int64_t rank_stride, int cols) {
    const int nv = k + 1 < nblocks ? QB : last_nv;
    const int ic = row < nv ? row : nv - 1;
    const int cc = 8 * ((lane % 8) ^ (row % 8));
    return (k * spb + (ic >> rs)) * step + (ic & (R - 1)) * rank_stride + (cc < cols ? cc : 0);
  };
  auto issue_x = [&](int64_t k, int slot) {
    const int64_t o = blk_off(k, 8 * w + lrow, xstep, P, ncol);
    dma16(x0 + o, xs_a + slot * PLANE + w * 1024);
    if constexpr (EPI) {
      if (has_z) dma16(z0 + o, zs_a + slot * PLANE + w * 1024);
    }
  };
  auto issue_bc = [&](int64_t k, int slot) {
#pragma unroll
    for (int jj = 0; jj < BC_PER; ++jj) {
      const int idx = w * BC_PER + jj;
      const bool isC = idx >= NPL * 8;
      const int rem = idx % (NPL * 8), pl = rem / 8, gr = rem % 8;
      const int col = pl * 64 + 8 * ((lane % 8) ^ lrow);
      if (col < Ni)
        dma16((isC ? C0 : B0) + blk_off(k, 8 * gr + lrow, bcstep, Nr, PB) + pl * 64,
              (isC ? cs_a : bs_a) + slot * BBLK + pl * PLANE + gr * 1024);
    }
  };
  auto issue_dl = [&](int64_t k, int slot) {
    const int nv = k + 1 < nblocks ? QB : last_nv;
    const int ic = lane < nv ? lane : nv - 1;
    const int64_t o = static_cast<int64_t>(ic >> rs) * H + k * spb * H;
    if (w == 4) dma2(d0 + o, dls_a + slot * QB * 4);
    if constexpr (TRAP) {
      if (w == 5) dma2(l0 + o, lls_a + slot * QB * 4);
    }
  };
  const int nxl = (EPI && has_z) ? 2 : 1;   // x (z) loads of a wave per block
  // loads of later blocks issued at the top of block k: delta (lam) of k + 3, B/C of k + 1, x (z) of k + 2;
  // returns the x (z) loads issued (they may stay in flight at the next top)
  auto issue_ahead = [&](int64_t k) {
    if (k + 3 < nblocks) issue_dl(k + 3, nxt(nxt(nxt(sd, NDS), NDS), NDS));
    if (k + 1 < nblocks) issue_bc(k + 1, nxt(sb, NBS));
    if (k + 2 < nblocks) {
      issue_x(k + 2, nxt(nxt(sx, NXS), NXS));
      return nxl;
    }
    return 0;
  };

  // ---- prologue (all waves): loads of blocks 0..2 in the order of three earlier iterations ----
  block_barrier();   // the zeroing is done before any load lands
  int vm_keep = 0;
  if (nblocks > 0) {
    issue_dl(0, 0);
    if (nblocks > 1) issue_dl(1, 1);
    issue_x(0, 0);
    if (nblocks > 2) issue_dl(2, 2);
    issue_bc(0, 0);
    if (nblocks > 1) {
      issue_x(1, 1);
      vm_keep = nxl;
    }
    wait_vm(vm_keep);
    block_barrier();
  }

// per-row arrays of block k, formed by state wave 0 during block k - 1 (the mask waves are the longer
// path through a block) and published by the barrier at the top of block k
  auto make_arrays = [&](int64_t k, int slot, int slot_next) {
    const int nv = k + 1 < nblocks ? QB : last_nv;
    const bool valid = lane < nv;
    const float d = valid ? __uint_as_float(dls[slot][lane] << 16) : 0.f;
    float v = (lane & (R - 1)) == 0 ? d * a2 : 0.f;   // the step's decay enters at its first row
    v += dppf<0x111, 0xf>(v);   // row_shr:1
    v += dppf<0x112, 0xf>(v);   // row_shr:2
    v += dppf<0x114, 0xf>(v);   // row_shr:4
    v += dppf<0x118, 0xf>(v);   // row_shr:8
    v += dppf<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
    v += dppf<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
    const float cs_end = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), kWave - 1));
    float wf = d, wd = d;
    if constexpr (TRAP) {
      const float lm = valid ? __uint_as_float(lls[slot][lane] << 16) : 0.f;
      // the next step's first row: in this block, or row 0 of the next block
      const int jn = (lane | (R - 1)) + 1;
      float dn = 0.f, ln = 0.f;
      if (jn < QB) {
        if (jn < nv) {
          dn = __uint_as_float(dls[slot][jn] << 16);
          ln = __uint_as_float(lls[slot][jn] << 16);
        }
      } else if (k + 1 < nblocks) {
        dn = __uint_as_float(dls[slot_next][0] << 16);
        ln = __uint_as_float(lls[slot_next][0] << 16);
      }
      wd = lm * d;
      wf = __builtin_fmaf(1.f - ln, dn, wd);
    }
    float* A_ = &arr[k & 1][0][0];
    A_[A_CS * QB + lane] = v;
    A_[A_ECS * QB + lane] = exp2_hw(v);
    A_[A_WF * QB + lane] = wf;
    A_[A_WD * QB + lane] = wd;
    A_[A_WL * QB + lane] = exp2_hw(cs_end - v) * wf;
  };

  if (!state_wave) {
    // =========================== mask waves ===========================

    // mask tiles: G^T = B . C^T for s tiles 0..3 and t tile pt, decayed and weighted; element v of s tile sj
    // is row s = 16 sj + 4 q + v, column t = 16 pt + lc.  Kept up to the diagonal (an earlier or the same
    // step), with the own-step weight on it (the same step); past the diagonal the exponent takes a bias
    // of -inf, so the element comes out 0 (a multiply by 0 could meet exp2 = inf there).
    // Only the ten tile pairs (t tile, s tile) with s <= t are nonzero (the rows of an s tile past t are
    // later steps); the other six stay at the zeros the set-up wrote.  They are shared out three per
    // mask wave, the last two waves repeating one of theirs (the same values written twice), so no wave
    // has more than three: wave pt takes pairs (tp[i], sp[i]).
    int tp[3], sp[3];
    switch (pt) {
      case 0: tp[0] = 3; sp[0] = 3; tp[1] = 3; sp[1] = 2; tp[2] = 3; sp[2] = 1; break;
      case 1: tp[0] = 3; sp[0] = 0; tp[1] = 2; sp[1] = 2; tp[2] = 2; sp[2] = 1; break;
      case 2: tp[0] = 2; sp[0] = 0; tp[1] = 1; sp[1] = 1; tp[2] = 1; sp[2] = 1; break;
      default: tp[0] = 1; sp[0] = 0; tp[1] = 0; sp[1] = 0; tp[2] = 0; sp[2] = 0; break;
    }
    // On a diagonal pair element v of a lane is kept where its s row's step is at most its t row's
    // (16 t is a multiple of R, so the test does not depend on the tile), with the own-step weight where
    // the two are the same step; past the diagonal the exponent takes a bias of -inf, so the element
    // comes out 0 (a multiply by 0 could meet exp2 = inf there).  Off the diagonal every element is kept.
    float dbias[4];
    uint32_t downm[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int ss = (4 * q + v) >> rs, st = lc >> rs;
      dbias[v] = ss <= st ? 0.f : -__builtin_inff();
      downm[v] = ss == st ? 0xffffffffu : 0u;
    }
    // 16-byte chunk (4 kb + q) of row 16 j + lc: the row tile part (16 j rows) and the plane (kb / 2) are
    // constants of each read
    int rd[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) rd[hh] = swz(lc, 4 * hh + q);
    // The mask is stored as M^T: row t, and within each 32-row k block the 8 s values a lane of group q
    // contracts, in the order of the X^T fragments (s = 32 kb + 16 (e / 4) + 4 q + e % 4 in slot 8 q + e)
    // G^T fragments of block k: C rows of t tile tp[i], B rows of s tile sp[i] (all reads issued first)
    struct GFrag { bf16x8 c[3][NKB], b[3][NKB]; };
    auto g_reads = [&](const GFrag*, int64_t) {
      GFrag f;
      const unsigned char* Bk = &bs[sb][0];
      const unsigned char* Ck = &cs_[sb][0];
#pragma unroll
      for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const int po = (kb / 2) * PLANE;
          f.c[i][kb] = lds_ld<bf16x8>(Ck, po + 16 * tp[i] * PROW + rd[kb % 2]);
          f.b[i][kb] = lds_ld<bf16x8>(Bk, po + 16 * sp[i] * PROW + rd[kb % 2]);
        }
      return f;
    };
    auto mask = [&](int64_t k, const GFrag& f) {
      const float* Au = &arr[k & 1][0][0];
      unsigned char* Mw = &ms[k & 1][0][0];
      f32x4 gacc[3];
#pragma unroll
      for (int i = 0; i < 3; ++i) gacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 3; ++i) gacc[i] = mfma16(f.b[i][kb], f.c[i][kb], gacc[i]);
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const bool diag = tp[i] == sp[i];
        const float ct = Au[A_CS * QB + 16 * tp[i] + lc];
        const int s0 = 16 * sp[i] + 4 * q;
        const float4 c4 = *reinterpret_cast<const float4*>(&Au[A_CS * QB + s0]);
        const float4 f4 = *reinterpret_cast<const float4*>(&Au[A_WF * QB + s0]);
        const float4 d4 = *reinterpret_cast<const float4*>(&Au[A_WD * QB + s0]);
        const float cc[4] = {c4.x, c4.y, c4.z, c4.w}, ff[4] = {f4.x, f4.y, f4.z, f4.w}, dd[4] = {d4.x, d4.y, d4.z, d4.w};
        float m[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint32_t own = diag ? downm[v] : 0u;
          const float e = exp2_hw((ct - cc[v]) + (diag ? dbias[v] : 0.f));
          const float wsel = __uint_as_float((own & __float_as_uint(dd[v])) | (~own & __float_as_uint(ff[v])));
          m[v] = gacc[i][v] * e * wsel;
        }
        // s tile sp = 2 kb + hh: chunk 4 kb + q of row t, bytes 8 hh .. +7; bf16 hi and lo parts
        const uint32_t h01 = pack2(m[0], m[1]), h23 = pack2(m[2], m[3]);
        const uint32_t l01 = pack2(m[0] - lo_f(h01), m[1] - hi_f(h01)), l23 = pack2(m[2] - lo_f(h23), m[3] - hi_f(h23));
        const int wo = 16 * tp[i] * PROW + (sp[i] >= 2 ? rd[1] : rd[0]) + 8 * (sp[i] & 1);
        *reinterpret_cast<u32x2*>(Mw + wo) = u32x2{h01, h23};
        *reinterpret_cast<u32x2*>(Mw + PLANE + wo) = u32x2{l01, l23};
      }
    };

    if (nblocks > 0) {
      for (int64_t k = 0; k < nblocks; ++k) {
        // outstanding may stay: the x (z) loads of block k + 1, issued after the B/C loads of block k
        wait_vm(vm_keep);
        block_barrier();
        // the mask's LDS reads first; this wave's loads of later blocks are issued while they are in flight
        const GFrag gf = g_reads(nullptr, k);
        __builtin_amdgcn_sched_barrier(0);
        vm_keep = issue_ahead(k);
        __builtin_amdgcn_sched_barrier(0);
        mask(k, gf);
        advance();
      }
      block_barrier();   // pairs with the state waves' last barrier
    }
    return;
  }

  // =========================== state waves ===========================
  // the state S^T, rows n = 16 i + 4 q + v, column p = p0 + 16 pt + lc
  const int64_t prow = p0 + 16 * pt + lc;
  const bool prow_ok = prow < P;                      // this lane's state column exists
  const bool scol_ok = p0 + 16 * pt + 4 * q < P;      // the four output columns this lane stores exist
  // output stores this wave issues per block: every lane's four columns lie past P in a wave whose first
  // column does (the slice is cut at a multiple of 8), and then the wave issues none
  const int nst = 16 * pt < ncol ? 4 : 0;
  f32x4 S[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int n0 = 16 * i + 4 * q;
    if (p.h0 != nullptr && n0 < Ni && prow_ok) {
      const float4 v = *reinterpret_cast<const float4*>(&p.h0[((b * H + h) * P + prow) * Nr + p.n0 + n0]);
      S[i] = f32x4{v.x, v.y, v.z, v.w};
    } else {
      S[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  // per-lane LDS offsets (the tile and plane parts of each read are constants)
  int rd[2];                       // 16-byte chunk 4 hh + q of row lc (C readout, mask reads)
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) rd[hh] = swz(lc, 4 * hh + q);
  // transposing reads: the lane points at row r4 = 4 q + lc / 4 (+ 16 u + 32 kb) and four columns from
  // 4 (lc % 4); X^T for columns 16 pt .., B^T for state tile i (columns 16 i ..)
  const int r4 = 4 * q + lc / 4;
  const int xt = r4 * PROW + (((2 * pt + (lc % 4) / 2) ^ (r4 & 7)) << 4) + 8 * (lc % 2);
  int bt[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) bt[i] = r4 * PROW + (((2 * i + (lc % 4) / 2) ^ (r4 & 7)) << 4) + 8 * (lc % 2);
  const int xo = swz(lc, 2 * pt + q / 2) + 8 * (q % 2);   // x at row lc of a tile, columns 16 pt + 4 q ..
  int64_t oo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = 16 * j + lc;
    oo[j] = static_cast<int64_t>(t >> rs) * xstep + (t & (R - 1)) * P + 16 * pt + 4 * q;
  }

  // one block on the state waves: the finish of block k - 1 (FIN), then block k's readout, X^T fragments and
  // state update.  Each phase issues all of its LDS reads before its first use, so their latencies overlap.
  auto step = [&](int64_t k, Carry& c, auto fin, int nv) {
    constexpr bool FIN = decltype(fin)::value;
    const unsigned char* Bk = &bs[sb][0];
    const unsigned char* Ck = &cs_[sb][0];
    const unsigned char* Xk = &xs[sx][0];
    const float* Au = &arr[k & 1][0][0];

    // -- reads: mask of block k - 1 (hi, lo) --
    bf16x8 mf[4][2][2];   // [row tile][k block][hi, lo]
    if constexpr (FIN) {
      const unsigned char* Mr = &ms[(k - 1) & 1][0][0];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          if (kb == 0 || j >= 2)
#pragma unroll
            for (int hl = 0; hl < 2; ++hl) mf[j][kb][hl] = lds_ld<bf16x8>(Mr, hl * PLANE + 16 * j * PROW + rd[kb]);
    }
    float ecs[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) ecs[j] = Au[A_ECS * QB + 16 * j + lc];
    __builtin_amdgcn_sched_barrier(0);

    // -- the state as A fragments in natural k order (slot e of lane group q is n = 32 kb + 8 q + e), split
    // into bf16 hi and lo parts: the accumulators hold rows 4 q + v of each tile, so two cross-lane swaps
    // regroup tiles 2 kb, 2 kb + 1 --
    bf16x8 sh[NKB], sl[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      uint32_t hw[4], lw[4];   // tile 2 kb rows (v0 v1, v2 v3), tile 2 kb + 1 rows (v0 v1, v2 v3)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int hv = 0; hv < 2; ++hv) {
          const float a = S[2 * kb + u][2 * hv], c2 = S[2 * kb + u][2 * hv + 1];
          const uint32_t hh = pack2(a, c2);
          hw[2 * u + hv] = hh;
          lw[2 * u + hv] = pack2(a - lo_f(hh), c2 - hi_f(hh));
        }
      auto regroup = [](const uint32_t (&v)[4]) {
        auto s0 = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
        auto s1 = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
        auto t0 = __builtin_amdgcn_permlane16_swap(s0[0], s0[1], false, false);
        auto t1 = __builtin_amdgcn_permlane16_swap(s1[0], s1[1], false, false);
        return __builtin_bit_cast(bf16x8, u32x4{t0[0], t1[0], t0[1], t1[1]});
      };
      sh[kb] = regroup(hw);
      sl[kb] = regroup(lw);
    }

    // -- finish of block k - 1: + X^T M^T, + D x, * silu(z), store --
    if constexpr (FIN) {
      uint16_t* const ob = PART ? nullptr : o0 + (k - 1) * spb * xstep;
      float* const pb = PART ? po0 + (k - 1) * spb * xstep : nullptr;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 acc = mfma16(c.xf0, mf[j][0][0], c.y[j]);
        acc = mfma16(c.xf0, mf[j][0][1], acc);
        if (j >= 2) {
          acc = mfma16(c.xf1, mf[j][1][0], acc);
          acc = mfma16(c.xf1, mf[j][1][1], acc);
        }
        float y[4] = {acc[0], acc[1], acc[2], acc[3]};
        if constexpr (EPI) {
          const u32x2 xv = c.xv[j];
          y[0] = __builtin_fmaf(Dh, lo_f(xv[0]), y[0]);
          y[1] = __builtin_fmaf(Dh, hi_f(xv[0]), y[1]);
          y[2] = __builtin_fmaf(Dh, lo_f(xv[1]), y[2]);
          y[3] = __builtin_fmaf(Dh, hi_f(xv[1]), y[3]);
          if (has_z) {
            const u32x2 zv = c.zv[j];
            const float zz[4] = {lo_f(zv[0]), hi_f(zv[0]), lo_f(zv[1]), hi_f(zv[1])};
#pragma unroll
            for (int v = 0; v < 4; ++v) y[v] *= zz[v] * __builtin_amdgcn_rcpf(1.f + exp2_hw(-zz[v] * kLog2e));
          }
        }
        if (scol_ok) {
          if constexpr (PART) *reinterpret_cast<float4*>(pb + oo[j]) = float4{y[0], y[1], y[2], y[3]};
          else *reinterpret_cast<u32x2*>(ob + oo[j]) = u32x2{pack2(y[0], y[1]), pack2(y[2], y[3])};
        }
      }
    }

    // -- reads: C of block k --
    bf16x8 cfr[4][NKB];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) cfr[j][kb] = lds_ld<bf16x8>(Ck, (kb / 2) * PLANE + 16 * j * PROW + rd[kb % 2]);
    __builtin_amdgcn_sched_barrier(0);

    // -- readout of the carried-in state for the four row tiles --
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        acc = mfma16(sh[kb], cfr[j][kb], acc);
        acc = mfma16(sl[kb], cfr[j][kb], acc);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[v] *= ecs[j];
      c.y[j] = acc;
    }
    __builtin_amdgcn_sched_barrier(0);

    // -- reads: X^T fragments (rows s = 32 kb + 16 (e / 4) + 4 q + e % 4 in slot e), x (z) at the output
    // points, the update weights and B^T --
    c.xf0 = cat(lds_tr(Xk, xt), lds_tr(Xk, xt + 16 * PROW));
    c.xf1 = cat(lds_tr(Xk, xt + 32 * PROW), lds_tr(Xk, xt + 48 * PROW));
    if constexpr (EPI) {
      const unsigned char* Zk = &zs[sx][0];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c.xv[j] = lds_ld<u32x2>(Xk, 16 * j * PROW + xo);
        c.zv[j] = lds_ld<u32x2>(Zk, 16 * j * PROW + xo);
      }
    }
    float4 wl[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) wl[kb][hf] = *reinterpret_cast<const float4*>(&Au[A_WL * QB + 32 * kb + 16 * hf + 4 * q]);
    const float dec = exp2_hw(Au[A_CS * QB + QB - 1]);
    bf16x8 btf[NT][2];
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int o = (i / 4) * PLANE + 32 * kb * PROW + bt[i % 4];
        btf[i][kb] = cat(lds_tr(Bk, o), lds_tr(Bk, o + 16 * PROW));
      }
    __builtin_amdgcn_sched_barrier(0);

    // -- state update: S^T = exp2(s_Q) S^T + B^T . Xw (Xw in bf16 hi and lo parts) --
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) S[i][v] *= dec;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const float4 w0 = wl[kb][0], w1 = wl[kb][1];
      const u32x4 xr = __builtin_bit_cast(u32x4, kb == 0 ? c.xf0 : c.xf1);
      const float xw[8] = {lo_f(xr[0]) * w0.x, hi_f(xr[0]) * w0.y, lo_f(xr[1]) * w0.z, hi_f(xr[1]) * w0.w,
                           lo_f(xr[2]) * w1.x, hi_f(xr[2]) * w1.y, lo_f(xr[3]) * w1.z, hi_f(xr[3]) * w1.w};
      bf16x8 xh, xl;
      split8(xw, xh, xl);
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        S[i] = mfma16(btf[i][kb], xh, S[i]);
        S[i] = mfma16(btf[i][kb], xl, S[i]);
      }
    }
    (void)nv;
  };

  // finish of the last block (its mask published)
  auto finish_last = [&](int64_t k, const Carry& c, int nv) {
    const unsigned char* Mr = &ms[k & 1][0][0];
    uint16_t* const ob = PART ? nullptr : o0 + k * spb * xstep;
    float* const pb = PART ? po0 + k * spb * xstep : nullptr;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x4 acc = mfma16(c.xf0, lds_ld<bf16x8>(Mr, 16 * j * PROW + rd[0]), c.y[j]);
      acc = mfma16(c.xf0, lds_ld<bf16x8>(Mr, PLANE + 16 * j * PROW + rd[0]), acc);
      if (j >= 2) {
        acc = mfma16(c.xf1, lds_ld<bf16x8>(Mr, 16 * j * PROW + rd[1]), acc);
        acc = mfma16(c.xf1, lds_ld<bf16x8>(Mr, PLANE + 16 * j * PROW + rd[1]), acc);
      }
      float y[4] = {acc[0], acc[1], acc[2], acc[3]};
      if constexpr (EPI) {
        const u32x2 xv = c.xv[j];
        y[0] = __builtin_fmaf(Dh, lo_f(xv[0]), y[0]);
        y[1] = __builtin_fmaf(Dh, hi_f(xv[0]), y[1]);
        y[2] = __builtin_fmaf(Dh, lo_f(xv[1]), y[2]);
        y[3] = __builtin_fmaf(Dh, hi_f(xv[1]), y[3]);
        if (has_z) {
          const u32x2 zv = c.zv[j];
          const float zz[4] = {lo_f(zv[0]), hi_f(zv[0]), lo_f(zv[1]), hi_f(zv[1])};
#pragma unroll
          for (int v = 0; v < 4; ++v) y[v] *= zz[v] * __builtin_amdgcn_rcpf(1.f + exp2_hw(-zz[v] * kLog2e));
        }
      }
      if (16 * j + lc < nv && scol_ok) {
        if constexpr (PART) *reinterpret_cast<float4*>(pb + oo[j]) = float4{y[0], y[1], y[2], y[3]};
        else *reinterpret_cast<u32x2*>(ob + oo[j]) = u32x2{pack2(y[0], y[1]), pack2(y[2], y[3])};
      }
    }
  };

  if (nblocks > 0) {
    if (w == 0) make_arrays(0, 0, 1);
    wait_vm(vm_keep);
    block_barrier();   // block 0's data and arrays: pairs with the top of the mask waves' block 0
    Carry c;
    vm_keep = issue_ahead(0);
    step(0, c, std::false_type{}, QB);
    if (w == 0) make_arrays(1, nxt(sd, NDS), nxt(nxt(sd, NDS), NDS));   // harmless past the last block
    advance();
    for (int64_t k = 1; k < nblocks; ++k) {
      // outstanding may stay: the x (z) loads of block k + 1 and the output stores of block k - 2 (four,
      // or none in a wave whose columns lie past the headdim), issued after the B/C loads of block k
      wait_vm(vm_keep + (k >= 2 ? nst : 0));
      block_barrier();   // block k's data and arrays, and block k - 1's mask, are in LDS
      vm_keep = issue_ahead(k);
      step(k, c, std::true_type{}, QB);
      if (w == 0) make_arrays(k + 1, nxt(sd, NDS), nxt(nxt(sd, NDS), NDS));   // harmless past the last block
      advance();
    }
    block_barrier();   // the last block's mask is complete
    finish_last(nblocks - 1, c, last_nv);
  }

  if (p.final_state != nullptr) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int n0 = 16 * i + 4 * q;
      if (n0 < Ni && prow_ok)
        *reinterpret_cast<float4*>(&p.final_state[((b * H + h) * P + prow) * Nr + p.n0 + n0]) =
            float4{S[i][0], S[i][1], S[i][2], S[i][3]};
    }
  }
}

template <int NP, bool TRAP, bool EPI, bool PART>
hipError_t launch_np(const SSDParams& sp, hipStream_t stream) {
  const int64_t blocks = sp.batch * sp.H * sp.nps;
  hipLaunchKernelGGL((ssd_kernel<NP, TRAP, EPI, PART>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                     stream, sp);
  return hipGetLastError();
}

template <int NP, bool TRAP>
hipError_t launch_gate(const SSDParams& sp, hipStream_t stream) {
  if (sp.part != nullptr) return launch_np<NP, TRAP, false, true>(sp, stream);
  const bool epi = sp.z != nullptr || sp.D != nullptr;
  return epi ? launch_np<NP, TRAP, true, false>(sp, stream) : launch_np<NP, TRAP, false, false>(sp, stream);
}

template <bool TRAP>
hipError_t launch_rule(const SSDParams& sp, hipStream_t stream) {
  return sp.N <= 64 ? launch_gate<64, TRAP>(sp, stream) : launch_gate<128, TRAP>(sp, stream);
}

// More than 128 states: the two shares of the state sum, then out = (share 0 + share 1 + D x) * silu(z).
// Four consecutive headdim columns per thread (P is a multiple of 64).
__global__ __launch_bounds__(256) void ssd_add_shares(const float* part, int64_t n_x, const uint16_t* x,
                                                      const uint16_t* z, const float* D, uint16_t* out,
                                                      int64_t RP, int64_t H) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= n_x) return;
  const float4 s0 = *reinterpret_cast<const float4*>(part + i);
  const float4 s1 = *reinterpret_cast<const float4*>(part + n_x + i);
  float y[4] = {s0.x + s1.x, s0.y + s1.y, s0.z + s1.z, s0.w + s1.w};
  if (D != nullptr) {
    const float Dh = D[(i / RP) % H];
    const u32x2 xv = *reinterpret_cast<const u32x2*>(x + i);
    y[0] = __builtin_fmaf(Dh, lo_f(xv[0]), y[0]);
    y[1] = __builtin_fmaf(Dh, hi_f(xv[0]), y[1]);
    y[2] = __builtin_fmaf(Dh, lo_f(xv[1]), y[2]);
    y[3] = __builtin_fmaf(Dh, hi_f(xv[1]), y[3]);
  }
  if (z != nullptr) {
    const u32x2 zv = *reinterpret_cast<const u32x2*>(z + i);
    const float zz[4] = {lo_f(zv[0]), hi_f(zv[0]), lo_f(zv[1]), hi_f(zv[1])};
#pragma unroll
    for (int v = 0; v < 4; ++v) y[v] *= zz[v] * __builtin_amdgcn_rcpf(1.f + exp2_hw(-zz[v] * kLog2e));
  }
  *reinterpret_cast<u32x2*>(out + i) = u32x2{pack2(y[0], y[1]), pack2(y[2], y[3])};
}

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

}  // namespace

bool ssd_supported(int64_t P, int64_t N) { return P % 8 == 0 && P > 0 && N % 16 == 0 && N > 0 && N <= 256; }
bool ssd_rank_supported(int64_t R) { return R == 1 || R == 2 || R == 4 || R == 8 || R == 16; }

// more than 128 states (one input per channel): the two shares of the state sum, fp32 [2][B, L, H, P]
size_t ssd_workspace_bytes(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int64_t, int64_t) {
  if (N <= 128) return 0;
  return align256(sizeof(float) * 2 * static_cast<size_t>(batch * L * H * P));
}

hipError_t ssd_launch(const SSDArgs& a, hipStream_t stream) {
  SSDParams sp{};
  sp.x = static_cast<const uint16_t*>(a.x);
  sp.delta = static_cast<const uint16_t*>(a.delta);
  sp.lam = static_cast<const uint16_t*>(a.lam);
  sp.A = a.A;
  sp.B = static_cast<const uint16_t*>(a.B);
  sp.C = static_cast<const uint16_t*>(a.C);
  sp.D = a.D;
  sp.z = static_cast<const uint16_t*>(a.z);
  sp.h0 = a.h0;
  sp.out = static_cast<uint16_t*>(a.out);
  sp.final_state = a.final_state;
  sp.batch = a.batch; sp.L = a.L; sp.H = a.H; sp.P = a.P; sp.N = a.N; sp.G = a.G;
  sp.R = static_cast<int>(a.R);
  sp.rs = 0;
  while ((1 << sp.rs) < sp.R) ++sp.rs;
  sp.nps = static_cast<int>((a.P + PB - 1) / PB);
  sp.Nr = a.N;
  sp.n0 = 0;
  sp.part = nullptr;
  auto run = [&](const SSDParams& q) { return a.lam != nullptr ? launch_rule<true>(q, stream) : launch_rule<false>(q, stream); };
  if (a.N <= 128) return run(sp);
  // states 0..127 and 128..N-1 as two shares (the sum over states is linear in them up to D x and the gate)
  const int64_t n_x = a.batch * a.L * a.H * a.P;
  float* part = static_cast<float*>(a.workspace);
  for (int s = 0; s < 2; ++s) {
    SSDParams q = sp;
    q.n0 = 128 * s;
    q.N = s == 0 ? 128 : a.N - 128;
    q.part = part + s * n_x;
    const hipError_t e = run(q);
    if (e != hipSuccess) return e;
  }
  if (n_x == 0) return hipSuccess;
  const int64_t blocks = (n_x / 4 + 255) / 256;
  hipLaunchKernelGGL(ssd_add_shares, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, part, n_x, sp.x,
                     sp.z, sp.D, sp.out, a.R * a.P, a.H);
  return hipGetLastError();
}

}  // namespace mssm
