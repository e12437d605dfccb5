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
// one (b, head, 64-wide headdim slice) and walks its sequence.  Wave w holds
// headdim columns 16 (w % 4).. of the transposed state S^T[n, p] for one half
// of the states (w / 4), in MFMA accumulators for the whole sequence, so the
// state never leaves the chip except as final_state.  Per block
// (v_mfma_f32_16x16x32_bf16, base-2 exponents, A pre-scaled by log2 e):
//   G^T = B . C^T   the 10 causal 16x16 tiles dealt out over the waves
//   M   = G o exp2(s_t - s_s) o w_s  ->  LDS, bf16 hi/lo pair, [t][s]
//   Y^T = exp2(s_t) (S . C^T) + X^T . M^T        (p x t; each wave of a pair reads
//                   out its half of the states for all row tiles, keeps two and
//                   hands the partner the other two through LDS)
//   S^T = exp2(s_Q) S^T + B^T . Xw               (n x p, k = rows)
// x, B and C enter the matrix cores exactly (bf16 inputs).  The three computed
// operands -- the state, the mask and the weighted inputs -- are each split
// into hi = bf16(v), lo = bf16(v - hi), about 16 significant bits.
//
// Data movement.  Every input reaches LDS by direct global->LDS loads
// (global_load_lds), in natural row-major order with each row's 16-byte
// chunks XOR-swizzled by the row index, so the reads below are free of bank
// conflicts: x two blocks ahead, B and C one block ahead, delta and lam three
// blocks ahead.  Fragments whose contraction index is the row index (B^T for
// the state update, X^T for the intra-block product) come from transposing
// LDS reads (ds_read_b64_tr_b16): in each 16-lane group, lane j receives
// element j of each of the four 4-element pieces that lanes 4k..4k+3 point
// at.  Each wave waits for its own loads (s_waitcnt vmcnt) and a barrier makes
// them visible; the compiler sees no loads into registers inside the loop, so
// nothing drains the prefetch.
#include <type_traits>

#include "internal.h"

namespace mssm {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kWave = 64;
constexpr int QB = 64;          // rows per block
constexpr int PB = 64;          // headdim slice per unit
constexpr int XROW = PB * 2;    // bytes of an x row in LDS (8 chunks of 16 bytes)
constexpr int XBLK = QB * XROW;
constexpr int MROW = (QB + 4) * 2;   // bytes of a mask row (padded: 16 rows hit distinct banks)
constexpr int MBLK = QB * MROW;
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
typedef __attribute__((address_space(3))) void lds_void;
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

// global -> LDS: lane l's 16 bytes land at lds_base + 16 l; a 2-byte load lands zero-extended in the
// dword at lds_base + 4 l.  lds_base is wave-uniform (it goes to M0).  Written as asm so that the
// compiler does not track these loads: it would otherwise wait for all of them before the transposing
// LDS reads of the same buffers, draining the prefetch; completion is waited for explicitly (wait_vm)
// before the barrier that publishes a block.  The asm has no outputs (the data goes to LDS), so no
// register can be overwritten while a load is in flight.
__device__ __forceinline__ uint32_t lds_addr(const unsigned char* p) {
  return __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)const_cast<unsigned char*>(p))));
}
__device__ __forceinline__ void dma16(const void* g, unsigned char* lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(lds_addr(lds_base)) : "memory", "m0");
}
__device__ __forceinline__ void dma2(const void* g, unsigned char* lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_ushort %0, off"
               :: "v"(g), "s"(lds_addr(lds_base)) : "memory", "m0");
}

// Barrier without a memory fence: LDS writes of this wave are complete
// first (lgkmcnt), direct loads were waited for by vmcnt before it.  The empty
// asm statements keep the compiler from moving LDS accesses across.
__device__ __forceinline__ void block_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// wait until at most n (0, 1 or 2; wave-uniform) of this wave's vector-memory operations are outstanding
__device__ __forceinline__ void wait_vm(int n) {
  if (n >= 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
  else if (n == 1) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
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
  int nps;       // headdim slices per head (P / 64)
};

// Causal G^T tiles (s-tile jt, t-tile it) handled by each of the 8 waves, packed (jt << 2) | it, -1 when
// none: waves 0 and 1 take two (a diagonal and an off-diagonal tile), the others one.  (A switch, so the
// choice is made with immediates: a table in memory would be a load inside the block loop.)
__device__ __forceinline__ int tile_of(int w, int k) {
  switch (w * 2 + k) {
    case 0: return 0x00; case 1: return 0x0b;
    case 2: return 0x05; case 3: return 0x03;
    case 4: return 0x0a;
    case 6: return 0x0f;
    case 8: return 0x01;
    case 10: return 0x06;
    case 12: return 0x02;
    case 14: return 0x07;
    default: return -1;
  }
}

constexpr int kWaves = 8;
constexpr int kThreads = kWave * kWaves;

// MFMA 16x16x32 lane layout: A row / B column = lane % 16, k slots 8(lane/16)..+7;
// accumulator element v of a lane is row 4 (lane / 16) + v, column lane % 16.
template <int NP, bool TRAP>
__global__ __launch_bounds__(kThreads) void ssd_kernel(SSDParams p) {
  static_assert(NP == 64 || NP == 128, "padded state count");
  constexpr int NTH = NP / 32;          // 16-row state tiles per wave (its half of the states)
  constexpr int NKH = NP / 64;          // 32-wide k blocks in a half
  constexpr int NKB = NP / 32;          // 32-wide k blocks over all states (C . B^T)
  constexpr int CPR = NP / 8;           // 16-byte chunks per B/C row
  constexpr int BROW = NP * 2;
  constexpr int BBLK = QB * BROW;
  constexpr int BC_PER_WAVE = 2 * CPR / kWaves;   // B then C, 64 / CPR rows per load
  static_assert(2 * CPR % kWaves == 0, "B/C loads split evenly over the waves");

  __shared__ __attribute__((aligned(16))) unsigned char xs[NXS][XBLK];
  __shared__ __attribute__((aligned(16))) unsigned char zs[NXS][XBLK];
  __shared__ __attribute__((aligned(16))) unsigned char bs[NBS][BBLK];
  __shared__ __attribute__((aligned(16))) unsigned char cs_[NBS][BBLK];
  __shared__ __attribute__((aligned(16))) uint32_t dls[NDS][QB];            // delta bits, one per row
  __shared__ __attribute__((aligned(16))) uint32_t lls[TRAP ? NDS : 1][QB];   // lam bits
  __shared__ __attribute__((aligned(16))) unsigned char ms[2][MBLK];         // mask hi / lo, [t][s]
  __shared__ __attribute__((aligned(16))) f32x4 xc[kWaves][2][kWave];        // partial readouts for the partner
  __shared__ __attribute__((aligned(16))) float arr[2][NARR][QB];
  static_assert(sizeof(xs) + sizeof(zs) + sizeof(bs) + sizeof(cs_) + sizeof(dls) + sizeof(lls) + sizeof(ms) +
                    sizeof(xc) + sizeof(arr) <= 160 * 1024,
                "LDS budget");

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform, in a scalar register
  const int pt = w % 4;                // 16-wide headdim tile of this wave
  const int nh = w / 4;                // half of the states it holds
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
  const int64_t L = p.L, H = p.H, P = p.P, N = p.N, G = p.G;
  const int R = p.R, rs = p.rs;
  const int Ni = static_cast<int>(N);
  const int spb = QB >> rs;            // steps per block
  const float a2 = p.A[h] * kLog2e;
  const float Dh = p.D != nullptr ? p.D[h] : 0.f;
  const bool has_z = p.z != nullptr;
  const int64_t nblocks = (L * R + QB - 1) / QB;
  const int last_nv = static_cast<int>(L * R - (nblocks - 1) * QB);   // rows of the last block

  // ---- zero what a load may leave untouched: B/C columns past N, mask tiles above the diagonal, and
  // whatever an earlier kernel left in the rings ----
  {
    unsigned char* regions[5] = {&xs[0][0], &zs[0][0], &bs[0][0], &cs_[0][0], &ms[0][0]};
    const int sizes[5] = {static_cast<int>(sizeof(xs)), static_cast<int>(sizeof(zs)), static_cast<int>(sizeof(bs)),
                          static_cast<int>(sizeof(cs_)), static_cast<int>(sizeof(ms))};
#pragma unroll
    for (int r = 0; r < 5; ++r)
      for (int e = tid * 16; e < sizes[r]; e += kThreads * 16)
        *reinterpret_cast<u32x4*>(regions[r] + e) = u32x4{0, 0, 0, 0};
  }

  // ---- per-lane offsets of the direct loads, fixed for the whole sequence (a block's are these plus the
  // block's first step times the step stride; the last block, when partial, recomputes them with its rows
  // clamped to its last valid row, whose weights are then 0) ----
  const int64_t xstep = H * R * P, bcstep = G * R * N;
  const uint16_t* const x0 = p.x + (b * L * H + h) * R * P + p0;         // step 0, rank 0 of this unit
  const uint16_t* const z0 = (has_z ? p.z : p.x) + (b * L * H + h) * R * P + p0;
  const uint16_t* const B0 = p.B + (b * L * G + g) * R * N;
  const uint16_t* const C0 = p.C + (b * L * G + g) * R * N;
  const uint16_t* const d0 = p.delta + b * L * H + h;
  const uint16_t* const l0 = TRAP ? p.lam + b * L * H + h : nullptr;
  uint16_t* const o0 = p.out + (b * L * H + h) * R * P + p0;
  auto x_off = [&](int nv) {   // this wave's x row group: rows 8w .. 8w + 7
    const int i = 8 * w + lane / 8;
    const int ic = i < nv ? i : nv - 1;
    const int c = (lane % 8) ^ (i % 8);   // logical chunk stored at this lane's physical chunk
    return static_cast<int64_t>(ic >> rs) * xstep + (ic & (R - 1)) * P + 8 * c;
  };
  int64_t bc_o[BC_PER_WAVE];
  bool bc_ok[BC_PER_WAVE];
  auto bc_off = [&](int nv) {
#pragma unroll
    for (int jj = 0; jj < BC_PER_WAVE; ++jj) {
      const int j = (w * BC_PER_WAVE + jj) % CPR;   // row group within B (first half) or C (second half)
      const int i = j * (kWave / CPR) + lane / CPR;
      const int ic = i < nv ? i : nv - 1;
      const int c = (lane % CPR) ^ (i % CPR);
      bc_ok[jj] = 8 * c < Ni;
      bc_o[jj] = static_cast<int64_t>(ic >> rs) * bcstep + (ic & (R - 1)) * N + 8 * c;
    }
  };
  auto dl_off = [&](int nv) {
    const int ic = lane < nv ? lane : nv - 1;
    return static_cast<int64_t>(ic >> rs) * H;
  };
  const int64_t xo_full = x_off(QB);
  const int64_t do_full = dl_off(QB);
  bc_off(QB);
  int64_t bo_full[BC_PER_WAVE];
#pragma unroll
  for (int jj = 0; jj < BC_PER_WAVE; ++jj) bo_full[jj] = bc_o[jj];

  // x (and z): one 1 KB load per wave per block (8 rows)
  auto issue_x = [&](int64_t k, int slot) {
    const int64_t o = (k + 1 < nblocks ? xo_full : x_off(last_nv)) + k * spb * xstep;
    dma16(x0 + o, &xs[slot][w * 1024]);
    if (has_z) dma16(z0 + o, &zs[slot][w * 1024]);
  };
  auto issue_bc = [&](int64_t k, int slot) {
    if (k + 1 == nblocks) bc_off(last_nv);
    const int64_t ko = k * spb * bcstep;
#pragma unroll
    for (int jj = 0; jj < BC_PER_WAVE; ++jj) {
      const int idx = w * BC_PER_WAVE + jj;
      const bool isC = idx >= CPR;
      const int j = idx % CPR;
      const int64_t o = (k + 1 == nblocks ? bc_o[jj] : bo_full[jj]) + ko;
      if (bc_ok[jj]) dma16((isC ? C0 : B0) + o, isC ? &cs_[slot][j * 1024] : &bs[slot][j * 1024]);
    }
  };
  // delta (and lam): one element per row, 2-byte loads into dword slots, by waves 0 (and 1)
  auto issue_dl = [&](int64_t k, int slot) {
    const int64_t o = (k + 1 < nblocks ? do_full : dl_off(last_nv)) + k * spb * H;
    if (w == 0) dma2(d0 + o, reinterpret_cast<unsigned char*>(&dls[slot][0]));
    if constexpr (TRAP) {
      if (w == 1) dma2(l0 + o, reinterpret_cast<unsigned char*>(&lls[slot][0]));
    }
  };

  // ---- per-row arrays of block k (wave 0) ----
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

  // ---- this wave's half of the state: S^T tiles, rows n = NP/2 nh + 16 i + 4 q + v, column p = p0 + 16 pt + lc
  const int64_t prow = p0 + 16 * pt + lc;
  const int nbase = (NP / 2) * nh;
  f32x4 S[NTH];
#pragma unroll
  for (int i = 0; i < NTH; ++i) {
    const int n0 = nbase + 16 * i + 4 * q;
    if (p.h0 != nullptr && n0 < Ni) {
      const float4 v = *reinterpret_cast<const float4*>(&p.h0[((b * H + h) * P + prow) * N + n0]);
      S[i] = f32x4{v.x, v.y, v.z, v.w};
    } else {
      S[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
#pragma unroll
  for (int i = 0; i < NTH; ++i) asm volatile("" : "+v"(S[i]));   // h0 has arrived before any direct load is issued

  // bit masks of the diagonal tile (fixed per lane): element v is row s = 4q + v, column t = lc of the
  // tile; it is kept up to the diagonal (an earlier or the same step), and takes the own-step weight on
  // it (the same step).  Bitwise selects: above the diagonal exp2(s_t - s_s) may overflow, and a
  // multiply by 0 would turn that into NaN.
  uint32_t keep[4], own[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int ss = (4 * q + v) >> rs, st = lc >> rs;
    keep[v] = ss <= st ? 0xffffffffu : 0u;
    own[v] = ss == st ? 0xffffffffu : 0u;
    asm volatile("" : "+v"(keep[v]), "+v"(own[v]));
  }

  // row tiles this wave finishes (the partner finishes the other two): {0, 3} or {1, 2}, equal causal work
  const int ja = nh == 0 ? 0 : 1, jb = nh == 0 ? 3 : 2;
  const int partner = w ^ 4;

  // ring slots, advanced by counters (no division in the loop)
  int sx = 0, sb = 0, sd = 0;   // slots of block k in the x, B/C and delta rings
  auto nxt = [](int v, int n) { return v + 1 == n ? 0 : v + 1; };

  // ---- prologue: loads of blocks 0..2 in the order of three earlier iterations ----
  block_barrier();   // the zeroing is done before any load lands
  int nx_prev = 0;
  if (nblocks > 0) {
    issue_dl(0, 0);
    if (nblocks > 1) issue_dl(1, 1);
    issue_x(0, 0);
    if (nblocks > 2) issue_dl(2, 2);
    issue_bc(0, 0);
    if (nblocks > 1) {
      issue_x(1, 1);
      nx_prev = has_z ? 2 : 1;
    }
    wait_vm(nx_prev);
    block_barrier();
    if (w == 0) make_arrays(0, 0, 1);
  }

  for (int64_t k = 0; k < nblocks; ++k) {
    const int nv = k + 1 < nblocks ? QB : last_nv;
    wait_vm(nx_prev);
    block_barrier();   // block k's data and arrays are in LDS; every wave is done with block k - 1
    {
      int s3 = nxt(nxt(nxt(sd, NDS), NDS), NDS), s2 = nxt(nxt(sx, NXS), NXS);
      if (k + 3 < nblocks) issue_dl(k + 3, s3);
      if (k + 1 < nblocks) issue_bc(k + 1, nxt(sb, NBS));
      nx_prev = 0;
      if (k + 2 < nblocks) {
        issue_x(k + 2, s2);
        nx_prev = has_z ? 2 : 1;
      }
    }
    const unsigned char* Bk = &bs[sb][0];
    const unsigned char* Ck = &cs_[sb][0];
    const unsigned char* Xk = &xs[sx][0];
    const float* Au = &arr[k & 1][0][0];

    // -- mask tiles: G^T = B . C^T (once per head), decayed and weighted --
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int tl = tile_of(w, kk);
      if (tl < 0) break;
      const int jt = tl >> 2, it = tl & 3;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      const int sr = 16 * jt + lc, tr = 16 * it + lc;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bf16x8 af = lds_ld<bf16x8>(Bk, sr * BROW + (((4 * kb + q) ^ (sr % CPR)) << 4));
        const bf16x8 bf = lds_ld<bf16x8>(Ck, tr * BROW + (((4 * kb + q) ^ (tr % CPR)) << 4));
        acc = mfma16(af, bf, acc);
      }
      const int t = 16 * it + lc, s0 = 16 * jt + 4 * q;
      const float ct = Au[A_CS * QB + t];
      const float4 c4 = *reinterpret_cast<const float4*>(&Au[A_CS * QB + s0]);
      const float4 f4 = *reinterpret_cast<const float4*>(&Au[A_WF * QB + s0]);
      float m[4] = {acc[0] * exp2_hw(ct - c4.x) * f4.x, acc[1] * exp2_hw(ct - c4.y) * f4.y,
                    acc[2] * exp2_hw(ct - c4.z) * f4.z, acc[3] * exp2_hw(ct - c4.w) * f4.w};
      if (jt == it) {
        const float4 d4 = *reinterpret_cast<const float4*>(&Au[A_WD * QB + s0]);
        const float wd[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int v = 0; v < 4; ++v) {   // same step: decay 1 and the own-step weight; later step: 0
          const uint32_t sel = (own[v] & __float_as_uint(acc[v] * wd[v])) | (~own[v] & __float_as_uint(m[v]));
          m[v] = __uint_as_float(sel & keep[v]);
        }
      }
      const uint32_t h01 = pack2(m[0], m[1]), h23 = pack2(m[2], m[3]);
      const uint32_t l01 = pack2(m[0] - lo_f(h01), m[1] - hi_f(h01));
      const uint32_t l23 = pack2(m[2] - lo_f(h23), m[3] - hi_f(h23));
      *reinterpret_cast<u32x2*>(&ms[0][t * MROW + 2 * s0]) = u32x2{h01, h23};
      *reinterpret_cast<u32x2*>(&ms[1][t * MROW + 2 * s0]) = u32x2{l01, l23};
    }

    // -- readout of the carried-in state over this wave's half, for all four row tiles; the two the
    // partner finishes go to it through LDS --
    bf16x8 sh[NKH], sl[NKH];   // state fragments (A: rows p, k = n in the accumulators' order)
#pragma unroll
    for (int kb = 0; kb < NKH; ++kb) {
      const float v[8] = {S[2 * kb][0], S[2 * kb][1], S[2 * kb][2], S[2 * kb][3],
                          S[2 * kb + 1][0], S[2 * kb + 1][1], S[2 * kb + 1][2], S[2 * kb + 1][3]};
      split8(v, sh[kb], sl[kb]);
    }
    f32x4 Ya, Yb;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 16 * j + lc;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKH; ++kb) {
        // C[t][n0 + 4q .. +3] and C[t][n0 + 16 + 4q .. +3] of this half's k block n0 = NP/2 nh + 32 kb
        const int cb = 4 * (NKH * nh + kb);
        const int c1 = cb + q / 2, c2 = cb + 2 + q / 2, off = 8 * (q % 2);
        const u32x2 a = lds_ld<u32x2>(Ck, t * BROW + ((c1 ^ (t % CPR)) << 4) + off);
        const u32x2 bb = lds_ld<u32x2>(Ck, t * BROW + ((c2 ^ (t % CPR)) << 4) + off);
        const bf16x8 cf = cat(a, bb);
        acc = mfma16(sh[kb], cf, acc);
        acc = mfma16(sl[kb], cf, acc);
      }
      const float e = Au[A_ECS * QB + t];
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[v] *= e;
      if (j == ja) Ya = acc;
      else if (j == jb) Yb = acc;
      else xc[w][(j == (nh == 0 ? 1 : 0)) ? 0 : 1][lane] = acc;   // the partner's tiles, in its order
    }

    // -- x^T fragments of this wave's columns (rows s = 32kb + 4q + k', +16): transposed reads --
    bf16x8 xf[2];
    {
      const int pc = 16 * pt + 4 * (lc % 4);    // column this lane points at
      const int off = 2 * (pc % 8);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int s1 = 32 * kb + 4 * q + lc / 4, s2 = s1 + 16;
        const u32x2 a = lds_tr(Xk, s1 * XROW + (((pc / 8) ^ (s1 % 8)) << 4) + off);
        const u32x2 bb = lds_tr(Xk, s2 * XROW + (((pc / 8) ^ (s2 % 8)) << 4) + off);
        xf[kb] = cat(a, bb);
      }
    }

    // -- state update of this half: S^T = exp2(s_Q) S^T + B^T . Xw --
    {
      const float dec = exp2_hw(Au[A_CS * QB + QB - 1]);
#pragma unroll
      for (int i = 0; i < NTH; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) S[i][v] *= dec;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const float4 w0 = *reinterpret_cast<const float4*>(&Au[A_WL * QB + 32 * kb + 4 * q]);
        const float4 w1 = *reinterpret_cast<const float4*>(&Au[A_WL * QB + 32 * kb + 16 + 4 * q]);
        const u32x4 xr = __builtin_bit_cast(u32x4, xf[kb]);
        const float xw[8] = {lo_f(xr[0]) * w0.x, hi_f(xr[0]) * w0.y, lo_f(xr[1]) * w0.z, hi_f(xr[1]) * w0.w,
                             lo_f(xr[2]) * w1.x, hi_f(xr[2]) * w1.y, lo_f(xr[3]) * w1.z, hi_f(xr[3]) * w1.w};
        bf16x8 xh, xl;
        split8(xw, xh, xl);
        const int s1 = 32 * kb + 4 * q + lc / 4, s2 = s1 + 16;
#pragma unroll
        for (int i = 0; i < NTH; ++i) {
          const int nc = nbase + 16 * i + 4 * (lc % 4);   // state column this lane points at
          const int off = 2 * (nc % 8);
          const u32x2 a = lds_tr(Bk, s1 * BROW + (((nc / 8) ^ (s1 % CPR)) << 4) + off);
          const u32x2 bb = lds_tr(Bk, s2 * BROW + (((nc / 8) ^ (s2 % CPR)) << 4) + off);
          const bf16x8 bt = cat(a, bb);
          S[i] = mfma16(bt, xh, S[i]);
          S[i] = mfma16(bt, xl, S[i]);
        }
      }
    }

    block_barrier();   // the mask and the partner's partial readouts are complete

    // -- finish two row tiles: + X^T M^T, + the partner's partial, + D x, * silu(z), store --
    const unsigned char* Mh = &ms[0][0];
    const unsigned char* Ml = &ms[1][0];
    const unsigned char* Zk = &zs[sx][0];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int j = kk == 0 ? ja : jb;
      f32x4 acc = kk == 0 ? Ya : Yb;
      const int t = 16 * j + lc;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (32 * kb <= 16 * j + 15) {
          const int o1 = t * MROW + 2 * (32 * kb + 4 * q), o2 = o1 + 32;
          const bf16x8 mh = cat(lds_ld<u32x2>(Mh, o1), lds_ld<u32x2>(Mh, o2));
          const bf16x8 mlo = cat(lds_ld<u32x2>(Ml, o1), lds_ld<u32x2>(Ml, o2));
          acc = mfma16(xf[kb], mh, acc);
          acc = mfma16(xf[kb], mlo, acc);
        }
      }
      const f32x4 o = xc[partner][kk][lane];
      if (t < nv) {
        const int pl = 16 * pt + 4 * q;   // first of this lane's 4 columns
        const int xo = t * XROW + (((pl / 8) ^ (t % 8)) << 4) + 2 * (pl % 8);
        const u32x2 xv = lds_ld<u32x2>(Xk, xo);
        float y[4] = {__builtin_fmaf(Dh, lo_f(xv[0]), acc[0] + o[0]), __builtin_fmaf(Dh, hi_f(xv[0]), acc[1] + o[1]),
                      __builtin_fmaf(Dh, lo_f(xv[1]), acc[2] + o[2]), __builtin_fmaf(Dh, hi_f(xv[1]), acc[3] + o[3])};
        if (has_z) {
          const u32x2 zv = lds_ld<u32x2>(Zk, xo);
          const float zz[4] = {lo_f(zv[0]), hi_f(zv[0]), lo_f(zv[1]), hi_f(zv[1])};
#pragma unroll
          for (int v = 0; v < 4; ++v) y[v] *= zz[v] * __builtin_amdgcn_rcpf(1.f + exp2_hw(-zz[v] * kLog2e));
        }
        const int64_t tt = k * spb + (t >> rs);
        const int r = t & (R - 1);
        *reinterpret_cast<u32x2*>(o0 + tt * xstep + r * P + pl) = u32x2{pack2(y[0], y[1]), pack2(y[2], y[3])};
      }
    }

    // -- the next block's per-row arrays (its delta and lam, and the step after it, arrived with this block) --
    const int sd1 = nxt(sd, NDS);
    if (w == 0 && k + 1 < nblocks) make_arrays(k + 1, sd1, nxt(sd1, NDS));
    sx = nxt(sx, NXS);
    sb = nxt(sb, NBS);
    sd = sd1;
  }

  if (p.final_state != nullptr) {
#pragma unroll
    for (int i = 0; i < NTH; ++i) {
      const int n0 = nbase + 16 * i + 4 * q;
      if (n0 < Ni)
        *reinterpret_cast<float4*>(&p.final_state[((b * H + h) * P + prow) * N + n0]) =
            float4{S[i][0], S[i][1], S[i][2], S[i][3]};
    }
  }
}

template <int NP, bool TRAP>
hipError_t launch_np(const SSDParams& sp, hipStream_t stream) {
  const int64_t blocks = sp.batch * sp.H * sp.nps;
  hipLaunchKernelGGL((ssd_kernel<NP, TRAP>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream, sp);
  return hipGetLastError();
}

}  // namespace

bool ssd_supported(int64_t P, int64_t N) { return P % PB == 0 && P > 0 && N % 16 == 0 && N > 0 && N <= 128; }
bool ssd_rank_supported(int64_t R) { return R == 1 || R == 2 || R == 4 || R == 8 || R == 16; }

size_t ssd_workspace_bytes(int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t) { return 0; }

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
  sp.nps = static_cast<int>(a.P / PB);
  if (a.lam != nullptr) {
    if (a.N <= 64) return launch_np<64, true>(sp, stream);
    return launch_np<128, true>(sp, stream);
  }
  if (a.N <= 64) return launch_np<64, false>(sp, stream);
  return launch_np<128, false>(sp, stream);
}

}  // namespace mssm
