// Grouped MFMA GEMM for the Newton-Schulz contractions on gfx950.
//
// One launch computes, for every unit u of a bucket chunk,
//     C_u = epilogue( L_u . R_u^T )      (TRANS = false: L_u (M x K) and
//                                         R_u (N x K) row-major, K contiguous)
//     C_u = epilogue( L_u^T . R_u )      (TRANS = true: L_u (K x M) and
//                                         R_u (K x N) row-major, K-major)
// The Newton-Schulz step of "Muon Optimizer and the Distributed
// Implementation" (section "Newton-Schulz Iteration"),
//     A = X X^T,   X' = a X + (b A + c A A) X = P X,   P = a I + b A + c A A,
// runs on the transposed copy Y = X^T (n x m) only: A = Y^T Y is a symmetric
// K-major product, P = c A A^T + b A + a I a symmetric row-major one (only
// upper-triangle tiles are computed, then mirrored), and the update is
// computed transposed, Y' = Y P^T (P is symmetric).
//
// Tiling (CDNA4, wave64): a workgroup of NW waves owns a BM x BN output tile
// (256 x 256, or 128 x 128 for small m); 2 x (NW / 2) waves each own (BM/2) x
// (2 BN / NW) built from 32x32 MFMA tiles (v_mfma_f32_32x32x16_{bf16,f16}; fp32
// issues four v_mfma_f32_32x32x2_f32 per 16-byte fragment).  NW = 4: one wave
// per SIMD, 128 x 128 accumulators in AGPRs; NW = 8: two waves per SIMD, 128 x
// 64 each (the compiler keeps them in VGPRs), so one wave's MFMAs can issue
// while the other waits on a memory instruction.
//
// Operand staging: K advances 128 bytes per row per stage (whole cache
// lines: the vector L1 keeps a bounded number of line requests in flight, so
// 128-byte pieces move twice the data of 64-byte ones).  Global -> LDS copies
// use buffer_load_dwordx4 ... lds (each lane's 16 bytes land at M0 + 16 *
// lane, 8 rows x 128 bytes per instruction), two stages in an LDS ring, so no
// registers hold staged data.  The 16-byte chunks of a row are XOR-swizzled
// with (row & 7) ^ ((row >> 3) & 1), which keeps the 32-row fragment reads
// free of bank conflicts for 8 and for 16 lanes per LDS cycle.  A K-major
// stage holds 64 K-rows of BM elements per operand, and fragments come out
// of it through ds_read_b64_tr_b16 (4 x 16 blocks read transposed).  Out-of-range
// rows and K chunks get an out-of-range buffer offset and read as zero; along
// K a 16-byte chunk is read when its first element is in range, which relies
// on leading dimensions that are multiples of 8 with zero padding (the
// workspace layout guarantees it).  Every operand matrix is smaller than 2^31
// bytes (checked by the planner).
//
// Schedule per stage (four k-steps of 16 bytes per lane half): the MFMAs of
// each step carry the fragment reads of the next; before the last step a
// barrier (after this wave's copies of the next stage landed and its reads
// of this stage completed) frees this stage's slot; the last step's MFMAs
// carry half of the copies of the stage after next into it (the other half
// ride on the first step of the next stage; 256 x 256 tiles) and the
// fragment reads of the next stage's first step.  A wave issues in order and an MFMA keeps the matrix pipe busy for
// 32 cycles, so each memory instruction is placed between two MFMAs.
//
// Epilogue: each wave stages its accumulators in LDS one 32-row strip at a
// time, reads the strip back as 16-byte row pieces, turns them into output
// values (scale; polynomial with the addend E read from global memory one
// strip ahead; or the fused parameter update, whose tile is a tile of the
// parameter block), and stores them as row chunks (direct pass, to C or the
// parameter) and/or transposed (mirror pass, to C2: the symmetric mirror).
// The strips are private to their wave: the passes synchronise the wave
// only, not the workgroup.
#pragma once

#include <type_traits>

#include "kernel_args.hpp"

namespace muon {

template <typename T> struct Mfma;

template <> struct Mfma<bf16> {
  static constexpr int NI = 1;  // MFMA instructions per 16-byte fragment pair
  __device__ __forceinline__ static void run(f32x16& acc, const u32x4& a, const u32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
};

template <> struct Mfma<f16> {
  static constexpr int NI = 1;
  __device__ __forceinline__ static void run(f32x16& acc, const u32x4& a, const u32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
  }
};

template <> struct Mfma<float> {
  static constexpr int NI = 4;
  __device__ __forceinline__ static void run(f32x16& acc, const u32x4& a, const u32x4& b) {
    // bit-cast the whole vector: a bit-cast of one vector-element lvalue
    // was lowered to element 0 for every e
    const f32x4 af = __builtin_bit_cast(f32x4, a);
    const f32x4 bf = __builtin_bit_cast(f32x4, b);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af[0], bf[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af[1], bf[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af[2], bf[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af[3], bf[3], acc, 0, 0, 0);
  }
};

// Buffer resource over [p, p + bytes): loads at offsets >= bytes return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t OOB = 0x80000000u;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt in bits 3:0
// and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// The same with lgkmcnt(0): this wave's LDS reads have completed as well.
template <int N> __device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4));
}

// 16 bytes per lane from global memory straight into LDS at dst + 16 * lane.
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t r, void* dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)dst, 16, off, 0, 0, 0);
}

// A wave-uniform pointer moved to scalar registers.
template <typename P> __device__ __forceinline__ P uniform_ptr(P p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return (P)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Upper-triangle tile t (row-major over bi <= bj) of a T x T tile grid.
__device__ __forceinline__ void upper_tile(int t, int T, int& bi, int& bj) {
  int i = 0;
  while (t >= T - i) {
    t -= T - i;
    ++i;
  }
  bi = i;
  bj = i + t;
}

// 8 consecutive elements of type T at p (16-byte aligned for 16-bit T,
// 32 bytes for fp32) <-> 8 floats.
template <typename T> __device__ __forceinline__ void load8(const T* p, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = to_f32(__builtin_bit_cast(T, (uint16_t)(w[e >> 1] >> ((e & 1) * 16))));
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[e + 4] = b[e]; }
  }
}

template <typename T> __device__ __forceinline__ void store8(T* p, const float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = pack2<T>(v[2 * j], v[2 * j + 1]);
    *as_global(reinterpret_cast<u32x4*>(p)) = w;
  } else {
    *as_global(reinterpret_cast<f32x4*>(p)) = f32x4{v[0], v[1], v[2], v[3]};
    *as_global(reinterpret_cast<f32x4*>(p + 4)) = f32x4{v[4], v[5], v[6], v[7]};
  }
}

// 8 consecutive elements of T stored through a buffer resource at byte
// offset off; an offset at or past the resource's size drops the store.
template <typename T>
__device__ __forceinline__ void buffer_store8(__amdgpu_buffer_rsrc_t r, uint32_t off, const float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = pack2<T>(v[2 * j], v[2 * j + 1]);
    __builtin_amdgcn_raw_buffer_store_b128(w, r, off, 0, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{v[0], v[1], v[2], v[3]}), r, off, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{v[4], v[5], v[6], v[7]}), r,
                                           off + 16, 0, 0);
  }
}

// 8 consecutive elements of T held as raw 16-byte words (one for 16-bit T,
// two for fp32), so that a strip's global loads can all be issued before the
// first one is used.
template <typename T> struct Raw8 {
  u32x4 w[sizeof(T) / 2];
};
template <typename T> __device__ __forceinline__ void raw_zero(Raw8<T>& r) {
#pragma unroll
  for (int h = 0; h < (int)(sizeof(T) / 2); ++h) r.w[h] = u32x4{0u, 0u, 0u, 0u};
}
template <typename T> __device__ __forceinline__ void raw_load8(const T* p, Raw8<T>& r) {
#pragma unroll
  for (int h = 0; h < (int)(sizeof(T) / 2); ++h) r.w[h] = reinterpret_cast<const u32x4*>(p)[h];
}
template <typename T> __device__ __forceinline__ void raw_unpack8(const Raw8<T>& r, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    const u32x4 w = r.w[0];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = to_f32(__builtin_bit_cast(T, (uint16_t)(w[e >> 1] >> ((e & 1) * 16))));
  } else {
    // whole-vector bit casts (a bit cast of one vector element lvalue was
    // lowered to element 0)
    const f32x4 lo = __builtin_bit_cast(f32x4, r.w[0]);
    const f32x4 hi = __builtin_bit_cast(f32x4, r.w[1]);
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[e] = lo[e]; v[e + 4] = hi[e]; }
  }
}

// Fused parameter update of 8 consecutive parameter elements (one row of the
// parameter block): W <- W (1 - lr wd) - lr scale O, or W <- O when
// store_only; O is also stored in fp32 when o is set.  final8_vec: all 8 in
// range, 16-byte aligned, the old W already loaded into raw; final8_tail:
// n_valid of them, element by element.
template <typename TW>
__device__ __forceinline__ void final8_vec(TW* w, float* o, const Raw8<TW>& raw, const float (&v)[8],
                                           float keep, float step, bool store_only) {
  float x[8];
  if (!store_only) {
    raw_unpack8<TW>(raw, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = x[e] * keep - step * v[e];
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = v[e];
  }
  store8(w, x);
  if (o) store8(o, v);
}

template <typename TW>
__device__ __forceinline__ void final8_tail(TW* w, float* o, const float (&v)[8], int n_valid, float keep,
                                            float step, bool store_only) {
  auto* wg = as_global(w);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (e < n_valid) {
      const float x = store_only ? v[e] : to_f32(wg[e]) * keep - step * v[e];
      wg[e] = from_f32<TW>(x);
      if (o) as_global(o)[e] = v[e];
    }
  }
}

// 4 x 16-bit transposed LDS read (ds_read_b64_tr_b16): within each group of
// 16 lanes, lane 4e + q supplies the address of 4 consecutive elements of
// row e, and lane L receives element L % 4 of the 4 lanes 4e + L / 4, e =
// 0..3, i.e. column 4 (L / 4) + L % 4 = L of rows 0..3: a 4 x 16 block read
// row-wise comes back column-wise (layout checked on the device).
// Issued as inline assembly: the compiler's builtin for it makes every such
// read wait for all outstanding LDS-DMA copies (it cannot tell the ring slots
// apart), which would serialize the copies of the next stage with the reads
// of this one.  The compiler does not track this read's completion, so the
// caller waits (lgkmcnt) before using the result.
__device__ __forceinline__ uint2 lds_read_tr16(const void* p) {
  uint2 r;
  const uint32_t addr = (uint32_t)(uintptr_t)(lds_ptr_t)p;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(addr));
  return r;
}

// The same with a constant byte offset: step kstep (0..7) of a K-major stage
// whose rows are ROWB bytes apart reads rows 16 (kstep / 2) + 4 (kstep % 2)
// further on, folded into the instruction's offset field.  The memory
// clobber keeps the compiler from moving LDS stores of the same wave past it.
template <int OFF> __device__ __forceinline__ uint2 lds_read_tr16_off(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  uint2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
}
template <int ROWB> __device__ __forceinline__ uint2 lds_read_tr16_step(uint32_t addr, int kstep) {
  switch (kstep) {
    case 0: return lds_read_tr16_off<0 * ROWB>(addr);
    case 1: return lds_read_tr16_off<4 * ROWB>(addr);
    case 2: return lds_read_tr16_off<16 * ROWB>(addr);
    case 3: return lds_read_tr16_off<20 * ROWB>(addr);
    case 4: return lds_read_tr16_off<32 * ROWB>(addr);
    case 5: return lds_read_tr16_off<36 * ROWB>(addr);
    case 6: return lds_read_tr16_off<48 * ROWB>(addr);
    default: return lds_read_tr16_off<52 * ROWB>(addr);
  }
}

// f(integral_constant<int, B>), ..., f(integral_constant<int, E - 1>), in order.
template <int B, int E, typename F> __device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// s_waitcnt lgkmcnt(0) alone.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// Orders this wave's LDS accesses before it against those after it, for the
// compiler (the fences, and the memory clobber for the transposed reads in
// inline asm) and the hardware (one wave's LDS instructions execute in
// issue order).  The epilogue's strips are private to their wave, so no
// other wave has to wait: against a workgroup barrier per strip pass this
// made the symmetric products 1-3% faster and the others 0.3-1.5%.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  asm volatile("" ::: "memory");
}

template <int BM, int BN, typename TI, typename TO, bool SYM, int EPI, bool TRANS = false, int NW = 4>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void gemm_kernel(const GemmArgs a) {
  constexpr int ES = (int)sizeof(TI);
  constexpr int EPC = 16 / ES;            // elements per 16-byte chunk
  constexpr int CPR = 8;                  // chunks per row per stage: 128 bytes, whole cache lines
  constexpr int BK = CPR * EPC;           // K elements per stage
  constexpr int NSTG = 2;                 // stages in the LDS ring
  constexpr int NSTEP = CPR / 2;          // MFMA k-steps per stage (one chunk per lane half)
  // NW waves: 2 along M by NW / 2 along N; NW / 2 of them copy each operand
  constexpr int WGN = NW / 2;             // waves along N
  constexpr int WPO = NW / 2;             // waves copying one operand
  constexpr int WTM = BM / 64;            // 32x32 tiles per wave along M (BM / 2 rows)
  constexpr int WN = BN / WGN;            // wave sub-tile width
  constexpr int WTN = WN / 32;            // 32x32 tiles per wave along N
  constexpr int STG = (BM + BN) * CPR;    // 16-byte slots per stage
  constexpr int NQ = STG / (64 * NW);     // copy instructions per wave per stage (8 rows each)
  constexpr int NDR = WTM + WTN;          // fragment reads per k-step
  constexpr int NPAIR = WTM * WTN;        // fragment pairs per k-step
  constexpr int CPP = (NQ + NPAIR - 1) / NPAIR;  // copies issued per MFMA pair
  constexpr int SROW = WN + 8;            // epilogue strip row stride (floats)
  static_assert(BM == BN, "square tiles");
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  static_assert(NQ * 8 * WPO == BM, "each wave copies 1 / WPO of one operand's rows");
  static_assert(NDR <= NPAIR, "fragment reads fit between the MFMAs of one step");
  static_assert(NW * 32 * SROW * 4 <= NSTG * STG * 16, "epilogue strips fit in the ring");

  __shared__ u32x4 ring[NSTG][STG];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: operand choice and buffer resource stay scalar
  const int wm = wid / WGN, wn = wid % WGN;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  // ---- workgroup -> (unit, tile).  Workgroup b runs on XCD b & 7.  Logical
  // tiles are dealt to the XCDs in chunks of S consecutive tiles, chunk c to
  // XCD c & 7: at any time the 8 XCDs work on neighbouring chunks (mostly one
  // unit, whose operands then stay in the Infinity Cache), and the ~32 tiles an
  // XCD runs at once lie in one chunk (operand bands shared through its L2).
  // S: 32 upper-triangle tiles for the K-major product, 64 for the row-major
  // symmetric ones (the polynomial, the Gram chain's m x m products), or two
  // 4-row groups of a non-symmetric product (measured best of 16..272, and
  // re-checked against 16/32/64 upper tiles and 4/16 groups as the kernels
  // changed).  The tail short of a full round of 8 chunks is split into 8
  // contiguous ranges, so the map stays a bijection.
  int logical;
  {
    const int b = blockIdx.x, tot = a.totalTiles;
    const int xcd = b & 7, loc = b >> 3;
    const int S = SYM ? (TRANS ? 32 : 64) : 8 * a.tilesN;
    const int full = tot / (8 * S);
    if (loc < full * S) {
      logical = (loc / S) * 8 * S + xcd * S + loc % S;
    } else {
      const int rest = tot - full * 8 * S, q = rest >> 3, r = rest & 7;
      logical = full * 8 * S + xcd * q + (xcd < r ? xcd : r) + (loc - full * S);
    }
  }
  // the division runs on the vector unit: bring the (uniform) results back
  // to scalar registers, or every buffer resource built from them would be
  // treated as divergent
  const int unit = __builtin_amdgcn_readfirstlane(logical / a.tilesPerUnit);
  const int tt = __builtin_amdgcn_readfirstlane(logical - unit * a.tilesPerUnit);
  int bi, bj;
  if constexpr (SYM) {
    upper_tile(tt, a.tilesM, bi, bj);
  } else {
    constexpr int GROUP = 4;
    const int per_group = GROUP * a.tilesN;
    const int g = tt / per_group;
    const int first = g * GROUP;
    const int gm = min(a.tilesM - first, GROUP);
    const int w = tt - g * per_group;
    bi = first + w % gm;
    bj = w / gm;
  }
  bi = __builtin_amdgcn_readfirstlane(bi);
  bj = __builtin_amdgcn_readfirstlane(bj);
  const int row0 = bi * BM, col0 = bj * BN;

  // chunk swizzle of a K-major stage.  16-bit: the transposed loads of 32
  // lanes read rows k..k+3 (k a multiple of 4) at 4 consecutive chunks each;
  // XOR with (0, 4, 10, 14)[k & 3] puts those 16 chunks on distinct 16-byte
  // bank groups of a 256-byte LDS cycle, and each 16-lane half on distinct
  // groups of a 128-byte one.  fp32: rows k and k+4 128 bytes apart.
  auto swz_t = [](int krow) {
    return ES == 2 ? (((krow & 1) << 2) ^ (((krow >> 1) & 1) * 10)) : ((krow >> 2) & 1) << 3;
  };

  // ---- copy plan: waves 0,1 copy L rows, waves 2,3 copy R rows, each wave
  // half of its operand's rows.  Copy q of a wave fills 64 consecutive slots
  // = 8 rows x 8 chunks; lane l lands in row 8q + l/8 (of the wave's half)
  // at physical chunk l % 8, which holds logical chunk (l % 8) ^ swz(row),
  // swz(row) = (row & 7) ^ ((row >> 3) & 1) = (l / 8) ^ (q & 1).
  const bool copiesL = wid < WPO;
  const TI* P = reinterpret_cast<const TI*>(copiesL ? a.L : a.R) +
                (int64_t)unit * (copiesL ? a.sL : a.sR);
  const int64_t ld = copiesL ? a.ldl : a.ldr;
  const int prows = copiesL ? a.M : a.N;
  const int cw = wid % WPO;  // this wave's share of its operand's rows
  const int slot_off = (copiesL ? 0 : BM * CPR) + cw * (BM / WPO) * CPR;
  // row-major operand (TRANS = false)
  const int crow = (copiesL ? row0 : col0) + cw * (BM / WPO) + (lane >> 3);  // operand row of copy 0
  const int ck0 = ((lane & 7) ^ (lane >> 3)) * EPC;        // k of this lane's chunk, even copies
  const int ck1 = ((lane & 7) ^ (lane >> 3) ^ 1) * EPC;    // odd copies
  const uint32_t cb0 = (uint32_t)(((int64_t)crow * ld + ck0) * ES);
  const uint32_t cb1 = (uint32_t)(((int64_t)crow * ld + ck1) * ES);
  const uint32_t cstep = (uint32_t)(8 * ld * ES);
  // K-major operand (TRANS): element (i, k) at P[k * ld + i].  A stage of an
  // operand is BK rows k of BM elements i, CR 16-byte chunks per row, chunk
  // c of row k at slot k * CR + (c ^ swzT(k)); a copy instruction fills 64
  // consecutive slots.
  constexpr int CR = BM * ES / 16;
  const int c0op = copiesL ? row0 : col0;
  const __amdgpu_buffer_rsrc_t rsrc =
      make_rsrc(P, (uint32_t)((int64_t)(TRANS ? a.K : prows) * ld * ES));
  // 16-bit K-major copies: copy q fills RPC K-rows; a lane's K-row and chunk
  // depend on q only through q & 1 (the chunk swizzle follows k & 3, and
  // 2 * NQ * RPC is a multiple of 4), so each lane keeps two base offsets,
  // and a copy adds the uniform part (q - (q & 1)) RPC + k0 rows.  Rows at or
  // past K fall outside the resource; a lane whose column is past the
  // operand starts at 2^31, past the resource at every stage (a wrap past
  // 2^32 in the zero-filled stages after the last one reaches only columns
  // whose output rows are dropped).
  constexpr int RPC = 64 / CR;  // K-rows per copy
  uint32_t tb[2] = {0u, 0u};
  if constexpr (TRANS && ES == 2) {
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int krow = (cw * NQ + par) * RPC + lane / CR;
      const int col = c0op + ((lane % CR) ^ swz_t(krow)) * EPC;
      tb[par] = col < prows ? (uint32_t)(((int64_t)krow * ld + col) * ES) : 0x80000000u;
    }
  }

  auto copy_one = [&](int q, int stage) {
    const int k0 = stage * BK;
    uint32_t off;
    if constexpr (TRANS && ES == 2) {
      off = tb[q & 1] + (uint32_t)(((int64_t)((q & ~1) * RPC + k0) * ld) * ES);
    } else if constexpr (TRANS) {
      const int slot = (cw * NQ + q) * 64 + lane;
      const int krow = slot / CR;
      const int lc = (slot % CR) ^ swz_t(krow);
      const int col = c0op + lc * EPC;
      const bool ok = (k0 + krow < a.K) && (col < prows);
      off = ok ? (uint32_t)(((int64_t)(k0 + krow) * ld + col) * ES) : OOB;
    } else {
      // rows past the operand fall outside the resource; a chunk past K
      // (which could reach into the next row) starts at 2^31, past it too.
      // The base depends on the stage and q & 1 only, so it is shared by
      // the copies of one stage.
      const int ck = (q & 1) ? ck1 : ck0;
      const uint32_t base = k0 + ck < a.K ? ((q & 1) ? cb1 : cb0) + (uint32_t)(k0 * ES) : 0x80000000u;
      off = base + (uint32_t)q * cstep;
    }
    copy16_to_lds(rsrc, &ring[stage % NSTG][slot_off + q * 64], off);
  };

  f32x16 acc[WTM][WTN];
#pragma unroll
  for (int i = 0; i < WTM; ++i)
#pragma unroll
    for (int j = 0; j < WTN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // fragments of one k-step (16 bytes per lane half), double buffered; the
  // fragment rows start at multiples of 32, so swz(row) depends on l32 only
  u32x4 fa[2][WTM], fb[2][WTN];
  const int rswz = (l32 & 7) ^ ((l32 >> 3) & 1);
  // K-major 16-bit: per-lane LDS byte address of fragment r's first
  // transposed read in stage slot 0 (lane 4e + q of each 16-lane group
  // addresses row 8 half + e at columns rb + 16 ((lane >> 4) & 1) + 4q; the
  // swizzle depends on the row only through e)
  constexpr int ROWB = CR * 16;
  uint32_t tbase[NDR];
  if constexpr (TRANS && sizeof(TI) == 2) {
    const int e = (lane >> 2) & 3, q = lane & 3;
    const uint32_t ring0 = (uint32_t)(uintptr_t)(lds_ptr_t)&ring[0][0];
#pragma unroll
    for (int r = 0; r < NDR; ++r) {
      const int region = r < WTM ? 0 : BM * CPR;
      const int rb = r < WTM ? wm * (BM / 2) + r * 32 : wn * WN + (r - WTM) * 32;
      const int col = rb + 16 * ((lane >> 4) & 1) + 4 * q;
      tbase[r] = ring0 + (uint32_t)(region * 16 + (8 * half + e) * ROWB + ((col >> 3) ^ swz_t(e)) * 16 +
                                    (col & 7) * 2);
    }
  }
  auto read_one = [&](int r, int stage, int s, int slot) {
    const u32x4* st = ring[stage % NSTG];
    const int region = r < WTM ? 0 : BM * CPR;                                    // L or R slots
    const int rb = r < WTM ? wm * (BM / 2) + r * 32 : wn * WN + (r - WTM) * 32;  // fragment's first row
    u32x4 v;
    if constexpr (!TRANS) {
      v = st[region + (rb + l32) * CPR + ((2 * s + half) ^ rswz)];
    } else if constexpr (sizeof(TI) == 2) {
      // 8 consecutive k (16s + 8 half + 0..7) of row rb + l32: two transposed
      // 4 x 16 reads, rows 16s + 4kq further on than the base address
      const uint32_t a0 = tbase[r] + (uint32_t)((stage % NSTG) * STG * 16);
#pragma unroll
      for (int kq = 0; kq < 2; ++kq) {
        const uint2 w = lds_read_tr16_step<ROWB>(a0, 2 * s + kq);
        v[2 * kq] = w.x;
        v[2 * kq + 1] = w.y;
      }
    } else {
      // fp32: 4 consecutive k (8s + 4 half + 0..3) of row rb + l32, one load each
      const int col = rb + l32;
      const float* base = reinterpret_cast<const float*>(st + region);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int krow = 8 * s + 4 * half + e;
        v[e] = __builtin_bit_cast(uint32_t, base[(krow * CR + ((col >> 2) ^ swz_t(krow))) * 4 + (col & 3)]);
      }
    }
    if (r < WTM) fa[slot][r] = v;
    else fb[slot][r - WTM] = v;
  };
  // p-th fragment read of a k-step (row-major operands): the fragment the
  // MFMA sequence (j fastest) needs p-th for the first time, A0, B0 ..
  // B(WTN-1), A1 .. A(WTM-1), so the next step's first MFMA waits for two
  // reads rather than for all of them (update and fused update 0.3-0.5%
  // faster).  K-major reads are all waited for at once and keep their order.
  auto ro = [](int p) { return TRANS ? p : (p == 0 ? 0 : (p <= WTN ? WTM + p - 1 : p - WTN)); };
  auto mfma_pair = [&](int p, int slot) {
    const int i = p / WTN, j = p % WTN;
    Mfma<TI>::run(acc[i][j], fa[slot][i], fb[slot][j]);
  };

  // 256 x 256 products split the copies of a stage: half go out during the
  // last step of the stage two before it (right after the barrier that frees
  // its slot), one every other MFMA; the other half during the first step of
  // the next stage, one per MFMA of its second half (the first half carries
  // the fragment reads).  All of them land before the barrier that precedes
  // that stage's last step.  Issuing all 16 copies back to back in one step
  // (one per MFMA) measured 4-5% slower on the update and on the K-major
  // product (spreading the second half over two steps: 0.5% slower than
  // this).
  constexpr bool SPLIT = NPAIR - NDR >= 8 && NQ == 16;
  constexpr int NQ3 = SPLIT ? NQ / 2 : NQ;
  constexpr int NQR = NQ - NQ3;
  static_assert(!SPLIT || (NQ3 * 2 <= NPAIR && NQR <= NPAIR - NDR), "split copy slots");

  const int nk = (a.K + BK - 1) / BK;
  // prologue: stage 0 and the first part of stage 1 in flight, then stage 0 visible
#pragma unroll
  for (int q = 0; q < NQ; ++q) copy_one(q, 0);
#pragma unroll
  for (int q = 0; q < NQ3; ++q) copy_one(q, 1);
  wait_vmcnt<NQ3>();
  __syncthreads();
#pragma unroll
  for (int r = 0; r < NDR; ++r) read_one(ro(r), 0, 0, 0);

  // transposed 16-bit reads are not tracked by the compiler: wait for them
  // explicitly before the MFMAs of the step they feed
  constexpr bool kManualLgkm = TRANS && sizeof(TI) == 2;
  for (int kt = 0; kt < nk; ++kt) {
    __builtin_amdgcn_sched_barrier(0);
    // steps 0 .. NSTEP-2: MFMAs on the fragments in registers, reads of the next step
#pragma unroll
    for (int s = 0; s + 1 < NSTEP; ++s) {
      if constexpr (kManualLgkm) wait_lgkm0();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int p = 0; p < NPAIR; ++p) {
        mfma_pair(p, s & 1);
        if (p < NDR) read_one(ro(p), kt, s + 1, (s + 1) & 1);
        if constexpr (SPLIT) {
          const int qq = s * (NPAIR - NDR) + (p - NDR);
          if (p >= NDR && qq < NQR) copy_one(NQ3 + qq, kt + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // this wave's copies of stage kt+1 landed and its fragment reads of
    // stage kt are done; after the barrier the same holds for every wave, so
    // stage kt's slot may be refilled
    wait_vmcnt_lgkm0<0>();
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    // last step: copies of stage kt+2 into the freed slot, fragment reads of
    // step 0 of stage kt+1
#pragma unroll
    for (int p = 0; p < NPAIR; ++p) {
      mfma_pair(p, (NSTEP - 1) & 1);
      if constexpr (SPLIT) {
        if ((p & 1) == 0 && p / 2 < NQ3) copy_one(p / 2, kt + 2);
      } else {
#pragma unroll
        for (int c = 0; c < CPP; ++c)
          if (p * CPP + c < NQ) copy_one(p * CPP + c, kt + 2);
      }
      if (p < NDR) read_one(ro(p), kt + 1, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---------------------------------------------------------------- epilogue
  wait_vmcnt_lgkm0<0>();  // the trailing (zero) copies and fragment reads are done
  __syncthreads();        // every wave is done with the ring
  float alpha = a.alpha;
  if (a.alphaSel != SEL_ONE) {
    const float4 ax = a.aux[unit];
    alpha *= a.alphaSel == SEL_INV_S ? ax.y : ax.z;
  }
  const TI* Ep = reinterpret_cast<const TI*>(a.E) + (int64_t)unit * a.sE;
  TO* Cp = a.C ? reinterpret_cast<TO*>(a.C) + (int64_t)unit * a.sC : nullptr;
  TO* C2p = a.C2 ? reinterpret_cast<TO*>(a.C2) + (int64_t)unit * a.sC2 : nullptr;
  // buffer resources of the outputs and the addend: a store at or past the
  // end is dropped, a load there returns zeros
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(Cp, (uint32_t)((int64_t)a.M * a.ldc * (int64_t)sizeof(TO)));
  const __amdgpu_buffer_rsrc_t c2rs = make_rsrc(C2p, (uint32_t)((int64_t)a.N * a.ldc2 * (int64_t)sizeof(TO)));
  const __amdgpu_buffer_rsrc_t ers = make_rsrc(Ep, (uint32_t)((int64_t)a.M * a.lde * ES));

  float keep = 1.f, step = 0.f;
  UnitDesc d;
  if constexpr (EPI == EPI_FINAL) {
    // the descriptor arrives through a vector load (this kernel stores to
    // global memory, so the compiler cannot prove a scalar load safe); its
    // fields are uniform: move them to scalar registers, or every buffer
    // resource built from them counts as divergent and each load of the old
    // parameter values runs in a waterfall loop
    d = a.desc[unit];
    d.w = uniform_ptr(d.w);
    d.o = uniform_ptr(d.o);
    d.ld = (int64_t)uniform_ptr((void*)(uintptr_t)d.ld);
    d.scale = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, d.scale)));
    keep = 1.f - a.lr * a.wd;
    step = a.lr * d.scale;
  }
  const bool store_only = a.finalMode == FINAL_STORE;
  const bool diag = SYM && bi == bj;
  // FINAL: the tile is a tile of the parameter block (O^T = Y P^T for a tall
  // unit, O = P X for a wide one), written by the direct pass
  const bool wpre = EPI == EPI_FINAL && !store_only && a.wvec != 0;
  const bool mirror = EPI != EPI_FINAL && C2p != nullptr;
  float* strip = reinterpret_cast<float*>(&ring[0][0]) + wid * (32 * SROW);
  // 16-bit outputs: the direct pass also leaves its converted values in a
  // 16-bit strip (rows RS16 bytes apart: the 4 rows a 16-lane transposed read
  // touches fall on distinct LDS banks), from which the mirror pass takes a
  // column's 8 values with two ds_read_b64_tr_b16: the mirror stores the very
  // bits of the direct pass, and reads 2 instructions instead of 8
  constexpr bool MIR16 = sizeof(TO) == 2;
  constexpr int RS16 = WN * 2 + 32;
  static_assert(NW * 32 * SROW * 4 + NW * 32 * RS16 <= NSTG * STG * 16, "16-bit strips fit in the ring");
  char* strip16 = reinterpret_cast<char*>(&ring[0][0]) + NW * 32 * SROW * 4 + wid * (32 * RS16);
  const int gc0 = col0 + wn * WN;  // global column of strip column 0

  // Each pass covers the 32 x WN strip of MFMA row-tile i in NT rounds of 64
  // lanes x 8 elements.  Direct pass: with CW = WN / 8 chunks per strip row,
  // lane l covers rows l / CW + (64 / CW) t at columns 8 (l % CW) .. +7.
  // Mirror pass: strip column jj, rows c8 .. c8 + 7.  16-bit: jj = 16 t +
  // l % 16, c8 = 8 (l / 16), so that the four 16-lane groups of a store (a
  // transposed read serves 16 columns at one c8) write the same 16 output
  // rows, 64 contiguous bytes each, instead of 64 rows of 16 bytes (the
  // polynomial and the Gram chain's products 2-3% faster).  fp32: jj =
  // (64 t + l) % WN, c8 = 8 ((64 t + l) / WN), conflict-free scalar reads.
  constexpr int NT = 32 * WN / 8 / 64;
  constexpr int CW = WN / 8, DRS = 64 / CW;
  static_assert(64 % CW == 0 && NT * DRS == 32, "direct pass covers the strip");
  const int dr0 = lane / CW, dc8 = (lane % CW) * 8;
  const int gj = gc0 + dc8;  // direct pass: this lane's first output column
  auto mpos = [&](int t, int& jj, int& c8) {
    if constexpr (MIR16) {
      jj = 16 * t + (lane & 15);
      c8 = 8 * (lane >> 4);
    } else {
      const int q = t * 64 + lane;
      jj = q % WN;
      c8 = (q / WN) * 8;
    }
  };

  // EPI_POLY's addend E at the direct-pass positions of strip i, as
  // unconditional buffer loads (pieces past column N get an out-of-range
  // offset).  Strip i + 1's loads are issued before strip i's stores, so
  // waiting for them never waits for a store.
  Raw8<TI> pe[2][NT];
  auto load_e = [&](int i, Raw8<TI>(&dst)[NT]) {
    const uint32_t estep = (uint32_t)(DRS * a.lde * ES);
    uint32_t off = gj < a.N ? (uint32_t)(((int64_t)(row0 + wm * (BM / 2) + i * 32 + dr0) * a.lde + gj) * ES) : OOB;
#pragma unroll
    for (int t = 0; t < NT; ++t, off += estep) {
#pragma unroll
      for (int h = 0; h < (int)(ES / 2); ++h) dst[t].w[h] = __builtin_amdgcn_raw_buffer_load_b128(ers, off + 16 * h, 0, 0);
    }
  };
  if constexpr (EPI == EPI_POLY) load_e(0, pe[0]);

  // EPI_FINAL: the old parameter values of strip i at the direct pass's
  // positions, loaded like E one strip ahead.  A per-strip buffer resource
  // starts at the strip's first parameter row, so offsets stay small
  // whatever the parameter's size; pieces not wholly inside the block stay
  // zero here and take the element-wise path, which reads W itself.
  Raw8<TO> pwb[2][NT];
  auto load_w = [&](int i, Raw8<TO>(&dst)[NT]) {
    const int prow0 = row0 + wm * (BM / 2) + i * 32;  // first parameter row of the strip
    // uniform, but the compiler clamps it with a vector instruction: back to
    // a scalar register, or the resource counts as divergent
    const int rows_in = __builtin_amdgcn_readfirstlane(max(0, min(32, a.M - prow0)));
    const TO* base = reinterpret_cast<const TO*>(d.w) + (int64_t)min(prow0, a.M) * d.ld;
    const __amdgpu_buffer_rsrc_t wrs = make_rsrc(base, (uint32_t)((int64_t)rows_in * d.ld * (int64_t)sizeof(TO)));
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int r = dr0 + DRS * t, c = gj;  // parameter row (from prow0) and first column of piece t
      const uint32_t off = wpre && c + 8 <= a.N ? (uint32_t)(((int64_t)r * d.ld + c) * (int64_t)sizeof(TO)) : OOB;
#pragma unroll
      for (int h = 0; h < (int)(sizeof(TO) / 2); ++h)
        dst[t].w[h] = __builtin_amdgcn_raw_buffer_load_b128(wrs, off + 16 * h, 0, 0);
    }
  };
  if constexpr (EPI == EPI_FINAL) load_w(0, pwb[0]);

  // one pass per MFMA row-tile i, with i a compile-time constant (a large
  // body can exceed the unroller's budget, and a run-time i would send the
  // accumulators to scratch memory)
  static_for<0, WTM>([&](auto ic) __attribute__((always_inline)) {
    constexpr int i = decltype(ic)::value;
    const int gr0 = row0 + wm * (BM / 2) + i * 32;  // global row of strip row 0

    Raw8<TO>(&pw)[NT] = pwb[i & 1];

    // accumulators of MFMA row-tile i -> strip[32][WN]
#pragma unroll
    for (int j = 0; j < WTN; ++j)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          strip[(g4 * 8 + half * 4 + r) * SROW + j * 32 + l32] = acc[i][j][g4 * 4 + r];
    wave_lds_sync();

    // final parameter update of 8 elements at (pr, pc..): vector form when the
    // row piece is whole and aligned, else element by element
    auto final8 = [&](const Raw8<TO>& raw, int pr, int pc, int ncols, const float (&v)[8]) {
      const int64_t off = (int64_t)pr * d.ld + pc;
      const int nv = min(8, ncols - pc);
      float* o = d.o ? d.o + off : nullptr;
      TO* w = reinterpret_cast<TO*>(d.w) + off;  // FINAL: TO is the parameter dtype
      if (a.wvec != 0 && nv == 8) final8_vec(w, o, raw, v, keep, step, store_only);
      else final8_tail(w, o, v, nv, keep, step, store_only);
    };

    // direct pass: all NT pieces are read before any is used, turned into
    // output values, written back when the mirror pass needs them, and
    // stored as 16-byte row chunks
    float v[NT][8];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float* sp = strip + (dr0 + DRS * t) * SROW + dc8;
      const f32x4 lo = *reinterpret_cast<const f32x4*>(sp);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(sp + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) { v[t][e] = lo[e]; v[t][e + 4] = hi[e]; }
    }
    if constexpr (EPI == EPI_FINAL) {
      if (i + 1 < WTM) load_w(i + 1, pwb[(i + 1) & 1]);
    }
    if constexpr (EPI == EPI_POLY) {
      if (i + 1 < WTM) load_e(i + 1, pe[(i + 1) & 1]);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int gi = gr0 + dr0 + DRS * t;
        float e8[8];
        raw_unpack8(pe[i & 1][t], e8);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          v[t][e] = alpha * v[t][e] + a.beta * e8[e] + (gi == gj + e ? a.gamma : 0.f);
      }
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) v[t][e] *= alpha;
    }
    if (mirror) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if constexpr (MIR16) {
          u32x4 w;
#pragma unroll
          for (int j = 0; j < 4; ++j) w[j] = pack2<TO>(v[t][2 * j], v[t][2 * j + 1]);
          *reinterpret_cast<u32x4*>(strip16 + (dr0 + DRS * t) * RS16 + dc8 * 2) = w;
        } else {
          float* sp = strip + (dr0 + DRS * t) * SROW + dc8;
          *reinterpret_cast<f32x4*>(sp) = f32x4{v[t][0], v[t][1], v[t][2], v[t][3]};
          *reinterpret_cast<f32x4*>(sp + 4) = f32x4{v[t][4], v[t][5], v[t][6], v[t][7]};
        }
      }
    }
    if constexpr (EPI == EPI_FINAL) {
      if (gj < a.N) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int gi = gr0 + dr0 + DRS * t;
          if (gi < a.M) final8(pw[t], gi, gj, a.N, v[t]);
        }
      }
    } else if (Cp) {
      if (!diag) {
        // rows at or past M fall outside the resource; pieces starting at or
        // past N (beyond the row's padding) get an out-of-range offset
        const uint32_t rstep = (uint32_t)(DRS * a.ldc * (int64_t)sizeof(TO));
        uint32_t off = gj < a.N ? (uint32_t)(((int64_t)(gr0 + dr0) * a.ldc + gj) * (int64_t)sizeof(TO)) : OOB;
#pragma unroll
        for (int t = 0; t < NT; ++t, off += rstep) buffer_store8<TO>(crs, off, v[t]);
      } else {
        // diagonal tile: the upper triangle (column >= row) is stored
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int gi = gr0 + dr0 + DRS * t;
          if (gi < a.M && gj < a.N && gi < gj + 8) {
            TO* dst = Cp + (int64_t)gi * a.ldc + gj;
            if (gi <= gj) {
              store8(dst, v[t]);
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (gi <= gj + e) dst[e] = from_f32<TO>(v[t][e]);
            }
          }
        }
      }
    }

    // mirror pass: strip column jj, rows c8..c8+7 -> row gc0 + jj of the
    // transposed output (rows of the output are the tile's columns, its
    // columns the tile's rows); all reads first, then the stores
    if (mirror && MIR16) {
      wave_lds_sync();  // values of the direct pass are in the 16-bit strip
      // a 16-lane group covers 16 consecutive strip columns jj at one c8;
      // lane 4e + q of it addresses row c8 + e (+4), columns 4q .. 4q + 3 of
      // the group, and receives its own column's 4 rows
      const int L = lane & 15;
      u32x4 mw[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        int jj, c8;
        mpos(t, jj, c8);
        const char* p = strip16 + (c8 + (L >> 2)) * RS16 + (jj - L + 4 * (L & 3)) * 2;
        const uint32_t addr = (uint32_t)(uintptr_t)(lds_ptr_t)p;
        const uint2 lo = lds_read_tr16_off<0>(addr);
        const uint2 hi = lds_read_tr16_off<4 * RS16>(addr);
        mw[t] = u32x4{lo.x, lo.y, hi.x, hi.y};
      }
      wait_lgkm0();  // the transposed reads are not tracked by the compiler
      if (!diag) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          int jj, c8;
          mpos(t, jj, c8);
          const int orow = gc0 + jj, ocol = gr0 + c8;
          // rows at or past N fall outside the resource
          const uint32_t off = ocol < a.M ? (uint32_t)(((int64_t)orow * a.ldc2 + ocol) * (int64_t)sizeof(TO)) : OOB;
          __builtin_amdgcn_raw_buffer_store_b128(mw[t], c2rs, off, 0, 0);
        }
      } else {
        // diagonal tile of a symmetric product: strictly lower positions
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          int jj, c8;
          mpos(t, jj, c8);
          const int orow = gc0 + jj, ocol = gr0 + c8;
          if (orow < a.N && ocol < a.M) {
            TO* dst = C2p + (int64_t)orow * a.ldc2 + ocol;
            if (ocol + 7 < orow) {
              *reinterpret_cast<u32x4*>(dst) = mw[t];
            } else {
              uint16_t* d16 = reinterpret_cast<uint16_t*>(dst);
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (ocol + e < orow) d16[e] = (uint16_t)(mw[t][e >> 1] >> (16 * (e & 1)));
            }
          }
        }
      }
    } else if (mirror) {
      wave_lds_sync();  // values of the direct pass are in the strip
      float mv[NT][8];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        int jj, c8;
        mpos(t, jj, c8);
#pragma unroll
        for (int e = 0; e < 8; ++e) mv[t][e] = strip[(c8 + e) * SROW + jj];
      }
      if (!diag) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          int jj, c8;
          mpos(t, jj, c8);
          const int orow = gc0 + jj, ocol = gr0 + c8;
          // rows at or past N fall outside the resource
          const uint32_t off = ocol < a.M ? (uint32_t)(((int64_t)orow * a.ldc2 + ocol) * (int64_t)sizeof(TO)) : OOB;
          buffer_store8<TO>(c2rs, off, mv[t]);
        }
      } else {
        // diagonal tile of a symmetric product: strictly lower positions
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          int jj, c8;
          mpos(t, jj, c8);
          const int orow = gc0 + jj, ocol = gr0 + c8;
          if (orow < a.N && ocol < a.M) {
            TO* dst = C2p + (int64_t)orow * a.ldc2 + ocol;
            if (ocol + 7 < orow) {
              store8(dst, mv[t]);
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (ocol + e < orow) dst[e] = from_f32<TO>(mv[t][e]);
            }
          }
        }
      }
    }
    wave_lds_sync();
  });
}

}  // namespace muon
