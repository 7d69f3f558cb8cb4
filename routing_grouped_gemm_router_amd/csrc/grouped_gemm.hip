// Grouped GEMM on CDNA4 matrix cores, bf16 (v_mfma_f32_32x32x16_bf16), fp8
// E4M3 with fp32 block scales (v_mfma_scale_f32_32x32x64_f8f6f4 at unit
// scale) and MXFP8 (the same instruction with the operands' E8M0 scales),
// fp32 accumulation: the experts' SwiGLU FFNs of "Scalable Training of
// Mixture-of-Experts Models with Megatron Core", section 2, Expert Computation
// (the local experts' GEMMs run together over their ragged row groups), and
// its section 5 low-precision recipes (blockwise FP8: 1 x 128 activation
// tiles, 128 x 128 weight blocks; MXFP8: 1 x 32 blocks).
//
//   forward  C[rows g]  = A[rows g] . B[g]       A [M,K]  B [G,K,N]
//   dgrad    dA[rows g] = dC[rows g] . B[g]^T    dC [M,N] B [G,K,N]
//   wgrad    dB[g]      = A[rows g]^T . dC[rows g]
//
// Design for gfx950:
//  * Two tile shapes, both with 64 x 64 per wave and two waves per SIMD (one
//    issues MFMAs while the other waits on LDS):
//      narrow: 128 x 128 tiles, 4 waves, two workgroups per CU, each with a
//              2-stage ring of 32 KiB stages;
//      wide:   128 x 256 tiles, 8 waves, one workgroup per CU with a 3-stage
//              ring of 48 KiB stages (two stages in flight while one is
//              consumed); a quarter less operand traffic per MFMA and half
//              again as many bytes in flight per CU.  Used whenever the
//              output width is a multiple of 256.
//    Persistent grid.  Each workgroup builds the per-group row-tile prefix
//    from the device offsets in LDS (no host sync), then walks the tiles: the
//    workgroups of one XCD take windows of consecutive tiles together, so
//    that a window's operand slabs are fetched into that XCD's L2 once.
//  * Operands go HBM -> LDS directly (buffer_load ... lds, 16 bytes per lane),
//    in slabs of 16 KiB (128 rows x 128 bytes); the ring runs across tile
//    boundaries: the next tile's first steps load during the current tile's
//    epilogue.  Buffer resources bound every tile's rows, so rows past a
//    group's end read as zero and nothing outside the operands is touched.
//  * Operands that are k-contiguous in memory are stored [row][k] (128 B rows)
//    and read with ds_read_b128; operands whose contraction axis is strided
//    (weights in the forward, both operands of wgrad) are stored as in memory,
//    [k][row] (256 B rows), and read with ds_read_b64_tr_b16, which hands each
//    lane four k values of its column.  16-byte chunks are XOR-swizzled by row
//    so that both the DMA writes and the fragment reads spread over all banks.
//  * Waves in a 2 x WN arrangement, each 64 x 64 = 2 x 2 MFMA 32x32x16 blocks,
//    issued as C^T = B^T A^T so that each lane holds 4 consecutive output
//    columns; the epilogue stages the wave's tile, 32 rows at a time, through
//    the ring slot just consumed and writes 16-byte vectors, 128 bytes per row.
//  * Epilogues: SwiGLU (AB and H = silu(A) * B from the fp32 sums; a tile holds
//    matching gate and up columns) and SwiGLU backward (dH -> dAB, reading AB).
//  * fp8: a k step is one 128-wide scale block.  Activations and gradients
//    arrive k-contiguous; the weights keep ONE code array in their own [K, N]
//    layout (a 128 x 128 block's scale serves both orientations), which the
//    data gradient reads k-contiguous and the forward as [k][column] slabs
//    through 8-bit transposing LDS reads.  Each step's MFMA partial is
//    promoted into the fp32 accumulator times the row scale of A and the row
//    scale of B, both DMA'd into LDS with the stage.
//  * MXFP8: every operand k-contiguous (its weight scales run along k, so the
//    weights keep one copy per orientation); each row's four E8M0 bytes of a stage (one
//    per 32 k) arrive as one dword DMA'd like the fp8 scales, and every lane
//    hands one block's byte to the MFMA, which applies both operands' scales
//    itself: the partials go straight into the accumulator.
#include "common.h"
#include "internal.h"

namespace moe {

#define LDS_AS __attribute__((address_space(3)))

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128;
constexpr int OP_BYTES = 16384;        // one operand slab of one stage: 128 rows x 128 bytes

// Tile shape: 2 x WN waves of 64 x 64; A is one slab, B is BN / 128 slabs.
template <int WN> struct Cfg {
  static constexpr int NW = 2 * WN;
  static constexpr int THREADS = 64 * NW;
  static constexpr int BN = 64 * WN;
  static constexpr int B_SLABS = BN / 128;
  static constexpr int STAGES = WN == 2 ? 2 : 3;
  static constexpr int WG_PER_CU = WN == 2 ? 2 : 1;
  static constexpr int A_PER = 16 / NW;            // DMA instructions per wave per stage, A
  static constexpr int B_PER = 16 * B_SLABS / NW;  // and B
  // fp8: row scales of A (128), then of B (BN); one 64-float vector per wave
  static constexpr int SCALE_BYTES = NW * 256;
};

// k elements per step: 128 bytes of each row
template <bool F8> struct KStep { static constexpr int value = F8 ? 128 : 64; };
template <int WN, bool F8> constexpr int stage_bytes() {
  return (1 + Cfg<WN>::B_SLABS) * OP_BYTES + (F8 ? Cfg<WN>::SCALE_BYTES : 0);
}
constexpr int MAX_GROUPS = 1024;
// tile patches: row-group modes (chunks of ROW_SN column tiles over all of a
// group's row tiles), weight gradient (WG_SM x WG_SN)
constexpr uint32_t ROW_SN = 4, WG_SM = 8, WG_SN = 4;
constexpr uint32_t RSRC_DW3 = 0x00020000u; // raw buffer, 32-bit elements, bounds-checked

enum Mode { FWD = 0, FWD_SWIGLU = 1, DGRAD = 2, DGRAD_SWIGLU_BWD = 3, WGRAD = 4 };
// operand precision: bf16, fp8 with fp32 block scales, MXFP8 (E8M0 per 32 k)
enum Prec { P_BF16 = 0, P_FP8 = 1, P_MX = 2 };

static int g_cu_count[64];

static int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (g_cu_count[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    g_cu_count[dev] = n;
  }
  return g_cu_count[dev];
}

__device__ __forceinline__ int64_t clamp64(int64_t v, int64_t lo, int64_t hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

// The lane id through an empty asm: values computed from it are recomputed
// where they are used instead of being hoisted out of the k loop, where
// they would hold registers across it.  The tile epilogues whose hoisted
// addresses pushed their kernel past 256 registers take it: the spill
// reloads inside the k loop then waited on vmcnt, i.e. on the stage's own
// prefetch DMA, and serialised the loads with the MFMAs.  Kernels that fit
// keep the plain lane id (recomputing there changed their schedule for the
// worse).
__device__ __forceinline__ int opaque_lane() {
  int v = static_cast<int>(threadIdx.x) & 63;
  asm volatile("" : "+v"(v));
  return v;
}

// chunk swizzles: KC layout [row][8 chunks], NC layout [k][16 chunks]
__device__ __forceinline__ int swz_kc(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz_nc(int kr) { return (kr & 3) << 2; }

typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer resource over [base, base + bytes): loads past the end return 0.
__device__ __forceinline__ i32x4_t make_rsrc(const void* base, uint64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t n = bytes > 0xffffffffull ? 0xffffffffu : static_cast<uint32_t>(bytes);
  i32x4_t r;
  r.x = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(a & 0xffffffffu));
  r.y = __builtin_amdgcn_readfirstlane(static_cast<int32_t>((a >> 32) & 0xffffu));
  r.z = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(n));
  r.w = static_cast<int32_t>(RSRC_DW3);
  return r;
}

// 16 bytes per lane from the buffer at byte offset voff into LDS at dst + 16 * lane.
// Issued as inline assembly so that the compiler adds no waits of its own: the
// ring is ordered by the explicit vmcnt waits and barriers below.
__device__ __forceinline__ void dma16(i32x4_t rs, LDS_AS void* dst, uint32_t voff) {
  const int32_t m0 = __builtin_amdgcn_readfirstlane(
      static_cast<int32_t>(reinterpret_cast<uintptr_t>(dst)));
  i32x4_t r;  // the descriptor must sit in scalar registers at the instruction
  r.x = __builtin_amdgcn_readfirstlane(rs.x);
  r.y = __builtin_amdgcn_readfirstlane(rs.y);
  r.z = __builtin_amdgcn_readfirstlane(rs.z);
  r.w = __builtin_amdgcn_readfirstlane(rs.w);
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(r), "s"(m0)
               : "memory", "m0");
}

// 4 bytes per lane into LDS at dst + 4 * lane (fp8 scale vectors)
__device__ __forceinline__ void dma4(i32x4_t rs, LDS_AS void* dst, uint32_t voff) {
  const int32_t m0 = __builtin_amdgcn_readfirstlane(
      static_cast<int32_t>(reinterpret_cast<uintptr_t>(dst)));
  i32x4_t r;
  r.x = __builtin_amdgcn_readfirstlane(rs.x);
  r.y = __builtin_amdgcn_readfirstlane(rs.y);
  r.z = __builtin_amdgcn_readfirstlane(rs.z);
  r.w = __builtin_amdgcn_readfirstlane(rs.w);
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(r), "s"(m0)
               : "memory", "m0");
}

// wait until this wave's DMA for the oldest in-flight stage has landed (at
// most n younger stages of PER instructions outstanding), then a workgroup
// barrier (no implicit fence: the DMA ring is ordered by vmcnt)
template <int PER>
__device__ __forceinline__ void wait_barrier(int n) {
  if (n <= 0)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Which tiles a workgroup takes.  Workgroup b runs on XCD b mod 8; the Q =
// P / 8 workgroups of one XCD take the Q consecutive tiles of a window
// together (so the window's operand slabs meet in that XCD's L2), and XCD x
// takes windows x, x + 8, x + 16, ...: at any time the XCDs work on
// neighbouring windows, which keeps their output writes close together in
// DRAM (starting the XCDs at different points of the list measured slower).
struct Walk {
  int64_t Q;   // workgroups per XCD (window size)
  int x, j;    // XCD, position inside the window
  int n;       // windows of this XCD
};

__device__ __forceinline__ Walk make_walk(int64_t total) {
  const int P = gridDim.x, b = blockIdx.x;
  Walk w;
  if (P % 8 == 0) {
    w.Q = P / 8;
    w.x = b % 8;
    w.j = b / 8;
    const int64_t W = (total + w.Q - 1) / w.Q;  // windows
    w.n = static_cast<int>(W > w.x ? (W - w.x + 7) / 8 : 0);
  } else {
    w.Q = P;
    w.x = 0;
    w.j = b;
    w.n = static_cast<int>((total + P - 1) / P);
  }
  return w;
}

// the next valid tile at or after step i of the walk; false once it is done
__device__ __forceinline__ bool walk_next(const Walk& w, int& i, int64_t total, int64_t& tau) {
  const int stride = w.Q == gridDim.x ? 1 : 8;
  for (; i < w.n; ++i) {
    tau = static_cast<int64_t>(w.x + stride * i) * w.Q + w.j;
    if (tau < total) return true;
  }
  return false;
}

struct Params {
  const char* A;   // element bytes: 2 (bf16) or 1 (fp8 codes)
  const char* B;
  const int64_t* off;
  int G;
  int64_t M;     // rows (row groups); contraction rows (wgrad; fp8: padded bound)
  int64_t Kc;    // contraction length (row groups) / K of dB (wgrad)
  int64_t Nout;  // product columns (row groups) / N of dB (wgrad)
  void* C;       // C, dA or dAB, or dB
  bf16_t* H;
  const bf16_t* ab;
  int out_f32;
  int accumulate;
  const float* sa;  // fp8 row scales of A: [Kc/128][M] (row groups), [M/128][Kc] (wgrad)
  const float* sb;  // fp8 row scales of B: [G][Kc/128][Nout] (row groups), [M/128][Nout] (wgrad)
  // MXFP8 E8M0 bytes, one per 32 contraction elements of each operand row:
  // A [M][Kc/32] and B [G][Nout][Kc/32] (row groups), A [Kc][ldm/32] and
  // B [Nout][ldm/32] (wgrad)
  const uint8_t* ea;
  const uint8_t* eb;
  int64_t ldm;      // fp8 wgrad: row length of the transposed operands
  // Routing weight applied inside the expert (row-group modes with SwiGLU):
  // forward H = row_scale[row] * silu(a) * b; backward dH = row_scale[row] *
  // dH' and gate_part[row, c] = sum over the 64 columns 64c.. of dH' * h.
  const float* row_scale;
  float* gate_part;
  // plain bf16 forward / dgrad: the 256-row and the 128-row kernels are both
  // launched and rows256_preferred picks the one that does the work
  int pair256;
};

// What a tile is: a ragged row block x 128 columns of one group (forward,
// dgrad), or a 128 x 128 block of one group's weight gradient (wgrad).
struct Tile {
  int g;
  int64_t row0;   // first output row (row groups) or first dB row (wgrad)
  int rows;       // valid output rows (row groups)
  int64_t nt;     // column tile
  int64_t lo;     // wgrad: first contraction row of the group
  int64_t nrows;  // wgrad: contraction rows of the group
  int nk;         // k steps (>= 1)
};

// Order of a group's tiles: blocks of up to SM row tiles; inside a block,
// chunks of SN column tiles, row-major inside a chunk.  The 32 consecutive
// tiles that one XCD's workgroups take at a time then form a compact patch
// (about 32 / SN row tiles x SN column tiles) wherever the run starts, so
// the patch's row slabs of A and column slabs of B are fetched into that
// XCD's L2 once.  Row-group modes use one block per group (SM = all of the
// group's row tiles).
template <uint32_t SN>
__device__ __forceinline__ void tile_in_group(uint32_t tl, uint32_t mt_g, uint32_t NT, uint32_t SM,
                                              uint32_t& m, uint32_t& n) {
  const uint32_t blk = tl / (SM * NT);
  const uint32_t r = tl - blk * SM * NT;
  const uint32_t sm = min(SM, mt_g - blk * SM);
  const uint32_t chunk = r / (sm * SN);
  const uint32_t rr = r - chunk * sm * SN;
  const uint32_t cw = min(SN, NT - chunk * SN);
  m = blk * SM + rr / cw;
  n = chunk * SN + rr % cw;
}

// Of a paired launch, the 256 x 256 tiling does the work when it needs at most
// 20/31 of the row tiles of the 128-row tiling (plain and SwiGLU epilogues),
// or at most 10/17 of them (SwiGLU backward).  A 256 x 256 tile costs about
// 1.8 times a 128 x 256 one and its ragged last tile rather less (a wave with
// no rows idles); over 256 groups with 7168 x 2048 and 4096 x 7168 weights
// the 256-row tiling of the plain epilogue measured faster at every tile
// ratio from 1.59 up and slower at 1.5 and below.  The SwiGLU forward ties at
// a ratio of 1.56 (256 groups) and is 10 % faster at about 1.8 (128 groups
// of 4096 x 3072); the SwiGLU backward is 6 % slower at 1.57, 9 % faster at
// 1.84 (the same 128 groups) and 12 % faster at 2 (one group of 8192 rows),
// a crossover near 1.7.  MXFP8 moves twice the FLOPs
// per operand byte of bf16, so its 128-row tiles are held back by the LDS
// DMA rate: the 256-row tiles ran 1.2 times faster per executed FLOP there,
// which pays for the larger ragged tails from a tile ratio of about 1.65 in
// every mode.
template <int MODE, int Q>
__device__ __forceinline__ bool rows256_preferred(int t128, int t256) {
  if (Q == P_MX) return 20LL * t128 >= 33LL * t256;
  if (MODE == DGRAD_SWIGLU_BWD) return 10LL * t128 >= 17LL * t256;
  return 20LL * t128 >= 31LL * t256;
}

// sum over the 64 lanes of a wave
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <int MODE, bool F8, int BN>
__device__ __forceinline__ bool decode(int64_t tau64, const Params& p, const int* s_pre,
                                       const int* s_off, int64_t NT64, int64_t total, Tile& t) {
  if (tau64 >= total) return false;
  const uint32_t tau = static_cast<uint32_t>(tau64), NT = static_cast<uint32_t>(NT64);
  if (MODE == WGRAD) {
    const uint32_t MT = static_cast<uint32_t>(p.Kc / BM);
    const uint32_t per_g = MT * NT;
    t.g = static_cast<int>(tau / per_g);
    uint32_t m, n;
    tile_in_group<WG_SN>(tau - static_cast<uint32_t>(t.g) * per_g, MT, NT, WG_SM, m, n);
    t.row0 = static_cast<int64_t>(m) * BM;
    t.nt = n;
    t.rows = BM;
    t.lo = s_off[t.g];
    t.nrows = s_off[t.g + 1] - t.lo;
    constexpr int BK = KStep<F8>::value;
    t.nk = t.nrows > 0 ? static_cast<int>((t.nrows + BK - 1) / BK) : 1;
  } else {
    // group g owns tiles [s_pre[g] * NT, s_pre[g+1] * NT)
    int glo = 0, ghi = p.G;
    while (ghi - glo > 1) {
      const int mid = (glo + ghi) >> 1;
      if (static_cast<uint32_t>(s_pre[mid]) * NT <= tau) glo = mid; else ghi = mid;
    }
    const int g = __builtin_amdgcn_readfirstlane(glo);
    t.g = g;
    const uint32_t base = static_cast<uint32_t>(s_pre[g]);
    const uint32_t mt_g = static_cast<uint32_t>(s_pre[g + 1]) - base;
    uint32_t m, n;
    tile_in_group<ROW_SN>(tau - base * NT, mt_g, NT, mt_g, m, n);
    const int64_t lo = s_off[g], hi = s_off[g + 1];
    t.row0 = lo + static_cast<int64_t>(m) * BM;
    t.nt = n;
    t.rows = static_cast<int>(min<int64_t>(BM, hi - t.row0));
    t.nk = static_cast<int>(p.Kc / KStep<F8>::value);
    t.lo = lo;
    t.nrows = hi - lo;
  }
  return true;
}

// Loader state of one tile: buffer resources and this lane's byte offsets
// for its 4 A and 4 B DMA instructions at k step 0, plus per-step deltas; for
// fp8 also the one scale-vector instruction of this wave.
template <int WN> struct Loader {
  i32x4_t ra, rb, rs;
  uint32_t va[Cfg<WN>::A_PER], vb[Cfg<WN>::B_PER], vs;
  uint32_t da, db, ds;
};

// Which operand layouts a mode uses in LDS: KC = [row][k] (k-contiguous in
// memory), otherwise [k][row] read by transposing.
template <int MODE, bool F8> struct Layout {
  static constexpr bool A_KC = F8 || MODE != WGRAD;
  static constexpr bool B_KC = F8 || MODE == DGRAD || MODE == DGRAD_SWIGLU_BWD;
};
// blockwise fp8 forward: B is the weight's own code layout [Kc, Nout], read
// in [k][column] slabs (MXFP8 keeps a k-contiguous copy: its scales run along k)
template <int MODE, int Q> constexpr bool fp8_b_nc() {
  return Q == P_FP8 && (MODE == FWD || MODE == FWD_SWIGLU);
}

// B-operand row of tile row rho (0..BN-1): the forward with SwiGLU pairs BN/2
// gate columns with the matching BN/2 up columns, 32 + 32 per wave
template <int MODE, int BN>
__device__ __forceinline__ int64_t b_row(const Tile& t, int rho, int64_t fh) {
  if (MODE == FWD_SWIGLU)
    return ((rho >> 5) & 1) * fh + t.nt * (BN / 2) + (rho >> 6) * 32 + (rho & 31);
  return t.nt * BN + rho;
}

// DMA instruction q of an operand (0 .. 16 x slabs - 1) fills 1 KiB of slab
// q / 16: in the [row][k] layout rows 8 (q % 16) .. + 7, in the [k][row] layout
// k rows 4 (q % 16) .. + 3.
template <int MODE, int Q, int WN>
__device__ __forceinline__ void setup_loader(const Params& p, const Tile& t, int wave, int lane,
                                             Loader<WN>& L) {
  using C = Cfg<WN>;
  constexpr bool F8 = Q != P_BF16;
  constexpr int BN = C::BN;
  constexpr int ES = F8 ? 1 : 2;  // element bytes
  constexpr int BK = KStep<F8>::value;
  const int64_t fh = p.Nout / 2;
  if (MODE == WGRAD && !F8) {
    // A = X [M, Kc] rows of the group, [k][row] layout; B = dC [M, Nout] likewise
    const int64_t K = p.Kc, N = p.Nout;
    L.ra = make_rsrc(p.A + t.lo * K * ES, static_cast<uint64_t>(t.nrows) * K * ES);
    L.rb = make_rsrc(p.B + t.lo * N * ES, static_cast<uint64_t>(t.nrows) * N * ES);
#pragma unroll
    for (int i = 0; i < C::A_PER; ++i) {
      const int q = wave * C::A_PER + i;
      const int kr = 4 * q + (lane >> 4), c = (lane & 15) ^ swz_nc(kr);
      L.va[i] = static_cast<uint32_t>((kr * K + t.row0 + 8 * c) * ES);
    }
#pragma unroll
    for (int i = 0; i < C::B_PER; ++i) {
      const int q = wave * C::B_PER + i, slab = q >> 4;
      const int kr = 4 * (q & 15) + (lane >> 4), c = (lane & 15) ^ swz_nc(kr);
      L.vb[i] = static_cast<uint32_t>((kr * N + t.nt * BN + slab * 128 + 8 * c) * ES);
    }
    L.da = static_cast<uint32_t>(BK * K * ES);
    L.db = static_cast<uint32_t>(BK * N * ES);
    return;
  }
  if (MODE == WGRAD && F8) {
    // A = X^T codes [Kc, ldm], B = dC^T codes [Nout, ldm]: rows of the tile,
    // contraction over the group's padded token range [lo, lo + nrows)
    const int64_t ldm = p.ldm;
    const bool any = t.nrows > 0;
    L.ra = make_rsrc(p.A + t.row0 * ldm + t.lo, any ? static_cast<uint64_t>(BM) * ldm : 0);
    L.rb = make_rsrc(p.B + t.nt * BN * ldm + t.lo, any ? static_cast<uint64_t>(BN) * ldm : 0);
#pragma unroll
    for (int i = 0; i < C::A_PER; ++i) {
      const int q = wave * C::A_PER + i;
      const int r = 8 * q + (lane >> 3), c = (lane & 7) ^ swz_kc(r);
      L.va[i] = static_cast<uint32_t>(r * ldm + c * 16);
    }
#pragma unroll
    for (int i = 0; i < C::B_PER; ++i) {
      const int q = wave * C::B_PER + i, slab = q >> 4;
      const int r = 8 * (q & 15) + (lane >> 3), c = (lane & 7) ^ swz_kc(r);
      L.vb[i] = static_cast<uint32_t>((slab * 128 + r) * ldm + c * 16);
    }
    L.da = L.db = 128;
    // waves past the A and B vectors repeat wave 0's load into their own
    // unused slot
    if (Q == P_MX) {
      // E8M0 [Kc][ldm/32] and [Nout][ldm/32]: dword lo/128 + kt of each row
      const int64_t nb = ldm / 32;
      const int64_t r = wave < 2 || wave >= 2 + 2 * C::B_SLABS
                            ? t.row0 + (wave < 2 ? wave : 0) * 64 + lane
                            : t.nt * BN + (wave - 2) * 64 + lane;
      const uint8_t* e = wave < 2 || wave >= 2 + 2 * C::B_SLABS ? p.ea : p.eb;
      const int64_t rows = wave < 2 || wave >= 2 + 2 * C::B_SLABS ? p.Kc : p.Nout;
      L.rs = make_rsrc(e, static_cast<uint64_t>(rows) * nb);
      L.vs = static_cast<uint32_t>(r * nb + t.lo / 32);
      L.ds = 4;
      return;
    }
    // scales [ldm/128][Kc] and [ldm/128][Nout], block lo/128 + kt
    const int64_t kb0 = t.lo / 128;
    if (wave < 2 || wave >= 2 + 2 * C::B_SLABS) {
      const int w = wave < 2 ? wave : 0;
      L.rs = make_rsrc(p.sa, static_cast<uint64_t>(ldm / 128) * p.Kc * 4);
      L.vs = static_cast<uint32_t>((kb0 * p.Kc + t.row0 + w * 64 + lane) * 4);
      L.ds = static_cast<uint32_t>(p.Kc * 4);
    } else {
      L.rs = make_rsrc(p.sb, static_cast<uint64_t>(ldm / 128) * p.Nout * 4);
      L.vs = static_cast<uint32_t>((kb0 * p.Nout + t.nt * BN + (wave - 2) * 64 + lane) * 4);
      L.ds = static_cast<uint32_t>(p.Nout * 4);
    }
    return;
  }
  // A: k-contiguous rows of the tile, [row][k] layout
  const int64_t Kc = p.Kc;
  L.ra = make_rsrc(p.A + t.row0 * Kc * ES, static_cast<uint64_t>(t.rows) * Kc * ES);
#pragma unroll
  for (int i = 0; i < C::A_PER; ++i) {
    const int q = wave * C::A_PER + i;
    const int r = 8 * q + (lane >> 3), c = (lane & 7) ^ swz_kc(r);
    L.va[i] = static_cast<uint32_t>(r * Kc * ES + c * 16);
  }
  L.da = 128;
  if (fp8_b_nc<MODE, Q>()) {
    // B = W_g codes [Kc, Nout]: slab q / 16 holds k rows 8 (q % 16) .. + 7 of
    // 128 columns, 128-byte rows with 16-byte chunks swizzled by k as in the
    // [row][k] layout; a chunk is 16 consecutive product columns
    const int64_t N = p.Nout;
    L.rb = make_rsrc(p.B + static_cast<int64_t>(t.g) * Kc * N, static_cast<uint64_t>(Kc) * N);
#pragma unroll
    for (int i = 0; i < C::B_PER; ++i) {
      const int q = wave * C::B_PER + i, slab = q >> 4;
      const int kr = 8 * (q & 15) + (lane >> 3), c = (lane & 7) ^ swz_kc(kr);
      L.vb[i] = static_cast<uint32_t>(kr * N + b_row<MODE, BN>(t, slab * 128 + 16 * c, fh));
    }
    L.db = static_cast<uint32_t>(128 * N);
  } else if (Layout<MODE, F8>::B_KC) {
    // B rows (output columns) are k-contiguous: bf16 dgrad W_g [Nout, Kc];
    // fp8 forward W_g^T codes [Nout, Kc]; fp8 dgrad W_g codes [Nout, Kc]
    const char* bg = p.B + static_cast<int64_t>(t.g) * p.Nout * Kc * ES;
    L.rb = make_rsrc(bg, static_cast<uint64_t>(p.Nout) * Kc * ES);
#pragma unroll
    for (int i = 0; i < C::B_PER; ++i) {
      const int q = wave * C::B_PER + i, slab = q >> 4;
      const int r = 8 * (q & 15) + (lane >> 3), c = (lane & 7) ^ swz_kc(r);
      L.vb[i] = static_cast<uint32_t>(b_row<MODE, BN>(t, slab * 128 + r, fh) * Kc * ES + c * 16);
    }
    L.db = 128;
  } else {
    // bf16 forward: B = W_g [Kc, Nout], [k][col] layout
    const int64_t N = p.Nout;
    L.rb = make_rsrc(p.B + static_cast<int64_t>(t.g) * Kc * N * ES, static_cast<uint64_t>(Kc) * N * ES);
#pragma unroll
    for (int i = 0; i < C::B_PER; ++i) {
      const int q = wave * C::B_PER + i, slab = q >> 4;
      const int kr = 4 * (q & 15) + (lane >> 4), c = (lane & 15) ^ swz_nc(kr);
      L.vb[i] = static_cast<uint32_t>((kr * N + b_row<MODE, BN>(t, slab * 128 + 8 * c, fh)) * ES);
    }
    L.db = static_cast<uint32_t>(BK * N * ES);
  }
  if (Q == P_MX) {
    // E8M0: A [M][Kc/32] rows of the tile (rows past the group read as zero
    // bytes, beside zero codes); B [G][Nout][Kc/32] at b_row(rho); dword kt of
    // each row; waves past the A and B vectors repeat wave 0's load
    const int64_t nb = Kc / 32;
    if (wave < 2 || wave >= 2 + 2 * C::B_SLABS) {
      const int w = wave < 2 ? wave : 0;
      L.rs = make_rsrc(p.ea + t.row0 * nb, static_cast<uint64_t>(t.rows) * nb);
      L.vs = static_cast<uint32_t>((w * 64 + lane) * nb);
    } else {
      L.rs = make_rsrc(p.eb + static_cast<int64_t>(t.g) * p.Nout * nb,
                       static_cast<uint64_t>(p.Nout) * nb);
      L.vs = static_cast<uint32_t>(b_row<MODE, BN>(t, (wave - 2) * 64 + lane, fh) * nb);
    }
    L.ds = 4;
  } else if (F8) {
    // scales: A [Kc/128][M] at row row0 + rho; B [G][Kc/128][Nout] at b_row(rho);
    // waves past the A and B vectors repeat wave 0's load into their own slot
    const int64_t nkb = Kc / 128;
    if (wave < 2 || wave >= 2 + 2 * C::B_SLABS) {
      const int w = wave < 2 ? wave : 0;
      L.rs = make_rsrc(p.sa, static_cast<uint64_t>(nkb) * p.M * 4);
      L.vs = static_cast<uint32_t>((t.row0 + w * 64 + lane) * 4);
      L.ds = static_cast<uint32_t>(p.M * 4);
    } else {
      L.rs = make_rsrc(p.sb + static_cast<int64_t>(t.g) * nkb * p.Nout,
                       static_cast<uint64_t>(nkb) * p.Nout * 4);
      L.vs = static_cast<uint32_t>(b_row<MODE, BN>(t, (wave - 2) * 64 + lane, fh) * 4);
      L.ds = static_cast<uint32_t>(p.Nout * 4);
    }
  }
}

template <bool F8, int WN>
__device__ __forceinline__ void issue(const Loader<WN>& L, int kt, LDS_AS char* stage, int wave) {
  using C = Cfg<WN>;
#pragma unroll
  for (int i = 0; i < C::A_PER; ++i)
    dma16(L.ra, stage + (wave * C::A_PER + i) * 1024, L.va[i] + kt * L.da);
#pragma unroll
  for (int i = 0; i < C::B_PER; ++i)
    dma16(L.rb, stage + OP_BYTES + (wave * C::B_PER + i) * 1024, L.vb[i] + kt * L.db);
  if (F8) dma4(L.rs, stage + (1 + C::B_SLABS) * OP_BYTES + wave * 256, L.vs + kt * L.ds);
}

// ---- fragment reads ----------------------------------------------------------

// [row][k] layout: 16 bytes of row r, chunk c
__device__ __forceinline__ u32x4_t chunk_kc(const LDS_AS char* op, int r, int c) {
  return *(const LDS_AS u32x4_t*)(op + r * 128 + ((c ^ swz_kc(r)) << 4));
}

__device__ __forceinline__ bf16x8_t frag_kc(const LDS_AS char* op, int r, int c) {
  return __builtin_bit_cast(bf16x8_t, chunk_kc(op, r, c));
}

// fp8 operand for one 32x32x64 MFMA: 32 k codes of row r (this lane's half
// of the 64), the same k positions for A and for B
__device__ __forceinline__ i32x8_t frag_kc8(const LDS_AS char* op, int r, int c0) {
  const u32x4_t lo = chunk_kc(op, r, c0), hi = chunk_kc(op, r, c0 + 1);
  const u32x4_t v[2] = {lo, hi};
  return __builtin_bit_cast(i32x8_t, v);
}

// fp8 [k][col] layout (128-byte rows of 128 columns, chunks swizzled by k as
// in the [row][k] layout): the 32 k codes k_base + 32 h .. + 31 of this lane's
// column, as four transposing reads of 8 k rows x 16 columns.  In each group
// of 16 lanes, lane j names row j / 2 and bytes 8 (j % 2) .. + 7 of the
// group's 16 columns, and receives column j's 8 codes in row order (checked
// with a one-wave probe of distinct byte values).
__device__ __forceinline__ i32x8_t frag_nc8(const LDS_AS char* op, int col_base, int k_base,
                                            int lane) {
  typedef int32_t i32x2_t __attribute__((ext_vector_type(2)));
  const int j = lane & 15;
  const int cc = (col_base >> 4) + ((lane >> 4) & 1);
  const int half = (j & 1) * 8;
  i32x2_t v[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int k = k_base + (lane >> 5) * 32 + 8 * r + (j >> 1);
    v[r] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (LDS_AS i32x2_t*)(op + k * 128 + ((cc ^ swz_kc(k)) << 4) + half));
  }
  return __builtin_bit_cast(i32x8_t, v);
}

// [k][col] layout: 8 k values (k0 .. k0+7 of this lane's half) of one column,
// with two transpose reads of 4 k x 16 columns each
__device__ __forceinline__ bf16x8_t frag_nc(const LDS_AS char* op, int col_base, int k_base,
                                            int lane) {
  const int i = lane & 15;
  const int col = col_base + ((lane >> 4) & 1) * 16 + 4 * (i & 3);
  const int k0 = k_base + (lane >> 5) * 8 + (i >> 2);
  const int cc = col >> 3, half = ((col >> 2) & 1) * 8;
  const LDS_AS char* p0 = op + k0 * 256 + ((cc ^ swz_nc(k0)) << 4) + half;
  const LDS_AS char* p1 = op + (k0 + 4) * 256 + ((cc ^ swz_nc(k0 + 4)) << 4) + half;
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4_t*)p0);
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4_t*)p1);
  const i16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

// opB points at the wave's B slab; wnl is the wave's 64-column half in it
template <int MODE>
__device__ __forceinline__ void compute_stage_bf16(f32x16_t (&acc)[2][2], const LDS_AS char* opA,
                                                   const LDS_AS char* opB, int wm, int wnl,
                                                   int lane) {
  constexpr bool A_NC = !Layout<MODE, false>::A_KC;
  constexpr bool B_NC = !Layout<MODE, false>::B_KC;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    bf16x8_t a[2], b[2];
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
      a[ii] = A_NC ? frag_nc(opA, wm * 64 + ii * 32, kk * 16, lane)
                   : frag_kc(opA, wm * 64 + ii * 32 + (lane & 31), kk * 2 + (lane >> 5));
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
      b[jj] = B_NC ? frag_nc(opB, wnl * 64 + jj * 32, kk * 16, lane)
                   : frag_kc(opB, wnl * 64 + jj * 32 + (lane & 31), kk * 2 + (lane >> 5));
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        acc[ii][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[jj], a[ii], acc[ii][jj], 0, 0, 0);
  }
}

// fp8: one 128-wide scale block per stage, as two MFMAs of 64 k per output
// block chained into one fp32 partial, which is then promoted once as
// acc += partial * scale_A(row) * scale_B(column) (the scales are constant
// over the block).  One promotion per 128 k halves the vector-ALU work per
// MFMA against promoting each 64-k half, and the first MFMA takes a zero
// accumulator operand, so the partial needs no clearing.
template <bool B_NC>
__device__ __forceinline__ void compute_stage_fp8(f32x16_t (&acc)[2][2], const LDS_AS char* opA,
                                                  const LDS_AS char* opB, const LDS_AS float* sA,
                                                  int wm, int wn, int wnl, int lane) {
  const LDS_AS float* sB = sA + BM;
  const int h = lane >> 5;
  float sa[2];
#pragma unroll
  for (int ii = 0; ii < 2; ++ii) sa[ii] = sA[wm * 64 + ii * 32 + (lane & 31)];
  i32x8_t a[2][2], b[2][2];  // [64-k half][block]
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
      a[s][ii] = frag_kc8(opA, wm * 64 + ii * 32 + (lane & 31), 4 * s + 2 * h);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
      b[s][jj] = B_NC ? frag_nc8(opB, wnl * 64 + jj * 32, 64 * s, lane)
                      : frag_kc8(opB, wnl * 64 + jj * 32 + (lane & 31), 4 * s + 2 * h);
  }
  const f32x16_t zero = {};
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    f32x4 sb[4];
#pragma unroll
    for (int vg = 0; vg < 4; ++vg) sb[vg] = *(const LDS_AS f32x4*)(sB + wn * 64 + jj * 32 + vg * 8 + h * 4);
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      // format 0 = E4M3 for both operands; E8M0 scale 127 = 1.0
      f32x16_t part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[0][jj], a[0][ii], zero, 0, 0,
                                                                      0, 127, 0, 127);
      part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[1][jj], a[1][ii], part, 0, 0, 0, 127,
                                                             0, 127);
#pragma unroll
      for (int vg = 0; vg < 4; ++vg)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[ii][jj][vg * 4 + e] += part[vg * 4 + e] * (sa[ii] * sb[vg][e]);
    }
  }
}

// MXFP8: the stage's 128 k are four 32-blocks; the dword of a row holds their
// E8M0 bytes, block b in byte b.  The scaled 32x32x64 MFMA splits its 64 k
// into two 32-blocks by byte position, not by lane half: bytes 0..15 of both
// halves form its first block, bytes 16..31 its second, and the scale of
// block j of a row comes from lane row + 32 j (measured with a one-wave probe
// of single non-zero codes under distinct per-lane scales).  So in step s
// lane half h loads the h-th 16 k of block 2 s into bytes 0..15 and the h-th
// 16 k of block 2 s + 1 into bytes 16..31, and passes the byte of block
// 2 s + h; the MFMA scales the products itself.
__device__ __forceinline__ i32x8_t frag_mx(const LDS_AS char* op, int r, int s, int h) {
  const u32x4_t lo = chunk_kc(op, r, 4 * s + h), hi = chunk_kc(op, r, 4 * s + 2 + h);
  const u32x4_t v[2] = {lo, hi};
  return __builtin_bit_cast(i32x8_t, v);
}

__device__ __forceinline__ void compute_stage_mx(f32x16_t (&acc)[2][2], const LDS_AS char* opA,
                                                 const LDS_AS char* opB, const LDS_AS uint32_t* eA,
                                                 int wm, int wn, int wnl, int lane) {
  const LDS_AS uint32_t* eB = eA + BM;
  const int h = lane >> 5;
  uint32_t xa[2], xb[2];
#pragma unroll
  for (int ii = 0; ii < 2; ++ii) xa[ii] = eA[wm * 64 + ii * 32 + (lane & 31)] >> (8 * h);
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) xb[jj] = eB[wn * 64 + jj * 32 + (lane & 31)] >> (8 * h);
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    i32x8_t a[2], b[2];
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) a[ii] = frag_mx(opA, wm * 64 + ii * 32 + (lane & 31), s, h);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) b[jj] = frag_mx(opB, wnl * 64 + jj * 32 + (lane & 31), s, h);
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        // format 0 = E4M3 for both; byte 0 of each scale operand is used
        acc[ii][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            b[jj], a[ii], acc[ii][jj], 0, 0, 0, static_cast<int>(xb[jj] >> (16 * s)), 0,
            static_cast<int>(xa[ii] >> (16 * s)));
  }
}

template <int MODE, int Q, int WN>
__device__ __forceinline__ void compute_stage(f32x16_t (&acc)[2][2], const LDS_AS char* stage,
                                              int wm, int wn, int lane) {
  const LDS_AS char* opA = stage;
  const LDS_AS char* opB = stage + OP_BYTES * (1 + (wn >> 1));
  if (Q == P_MX)
    compute_stage_mx(acc, opA, opB,
                     (const LDS_AS uint32_t*)(stage + (1 + Cfg<WN>::B_SLABS) * OP_BYTES), wm, wn,
                     wn & 1, lane);
  else if (Q == P_FP8)
    compute_stage_fp8<fp8_b_nc<MODE, Q>()>(acc, opA, opB,
                      (const LDS_AS float*)(stage + (1 + Cfg<WN>::B_SLABS) * OP_BYTES), wm, wn,
                      wn & 1, lane);
  else
    compute_stage_bf16<MODE>(acc, opA, opB, wm, wn & 1, lane);
}

// ---- epilogue ------------------------------------------------------------------
// acc[ii][jj][v] = C[m][n], m = wm*64 + ii*32 + (lane & 31),
//                          n = wn*64 + jj*32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3).
// Staging per wave: 4 KiB = [32 m][64 n] bf16 (128 B rows, chunks swizzled by
// m & 7), one half (ii) of the wave's rows at a time.

__device__ __forceinline__ uint32_t pack2(float a, float b) { return f32x2_to_bf16x2(a, b); }

__device__ __forceinline__ int stg_off(int m, int chunk) { return m * 128 + ((chunk ^ (m & 7)) << 4); }

// write rows ii*32 .. ii*32+31 of the wave's acc into staging as bf16
__device__ __forceinline__ void stage_acc(LDS_AS char* stg, const f32x16_t (&acc)[2][2], int ii,
                                          int lane) {
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int vg = 0; vg < 4; ++vg) {
      const int m = lane & 31;
      const int n = jj * 32 + vg * 8 + (lane >> 5) * 4;
      u32x2_t w;
      w.x = pack2(acc[ii][jj][vg * 4 + 0], acc[ii][jj][vg * 4 + 1]);
      w.y = pack2(acc[ii][jj][vg * 4 + 2], acc[ii][jj][vg * 4 + 3]);
      *(LDS_AS u32x2_t*)(stg + stg_off(m, n >> 3) + (n & 7) * 2) = w;
    }
}

__device__ __forceinline__ void unpack8(const uint4& v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
  return make_uint4(pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7]));
}

template <int MODE, int BN>
__device__ __forceinline__ void epilogue(const Params& p, const Tile& t, const f32x16_t (&acc)[2][2],
                                         LDS_AS char* stg, int wm, int wn, int lane) {
  const int rows_w = MODE == WGRAD ? 64 : t.rows - wm * 64;  // valid rows of this wave
  if (rows_w <= 0) return;
  if (MODE == WGRAD && p.out_f32) {
    // direct 16-byte stores of 4 consecutive fp32 columns
    float* out = static_cast<float*>(p.C) + static_cast<int64_t>(t.g) * p.Kc * p.Nout;
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int vg = 0; vg < 4; ++vg) {
          const int64_t m = t.row0 + wm * 64 + ii * 32 + (lane & 31);
          const int64_t n = t.nt * BN + wn * 64 + jj * 32 + vg * 8 + (lane >> 5) * 4;
          float4* q = reinterpret_cast<float4*>(out + m * p.Nout + n);
          float4 v = make_float4(acc[ii][jj][vg * 4], acc[ii][jj][vg * 4 + 1],
                                 acc[ii][jj][vg * 4 + 2], acc[ii][jj][vg * 4 + 3]);
          if (p.accumulate) {
            const float4 o = *q;
            v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
          }
          *q = v;
        }
    return;
  }
  const int64_t fh = p.Nout / 2;
#pragma unroll
  for (int ii = 0; ii < 2; ++ii) {
    if (ii * 32 >= rows_w) break;
    const bool store_c = MODE != FWD_SWIGLU || p.C != nullptr;
    if (store_c) {
      stage_acc(stg, acc, ii, lane);
      // 32 rows x 8 chunks; lane handles chunks lane + 64 i
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int idx = lane + 64 * i;
        const int m = idx >> 3, c = idx & 7;
        const bool valid = ii * 32 + m < rows_w;
        if (MODE == DGRAD_SWIGLU_BWD && p.row_scale) {
          // gated: dH = w dH', and the partial <dH', h> of this row over the
          // wave's 64 columns (8 consecutive lanes hold the row's 8 chunks)
          const u32x4_t vv = *(const LDS_AS u32x4_t*)(stg + stg_off(m, c));
          const int64_t row = t.row0 + wm * 64 + ii * 32 + m;
          const int64_t col = t.nt * BN + wn * 64 + 8 * c;
          const int64_t w2 = 2 * p.Nout;
          float dot = 0.0f;
          if (valid) {
            float dh[8], a[8], b[8], da[8], db[8];
            unpack8(make_uint4(vv.x, vv.y, vv.z, vv.w), dh);
            unpack8(*reinterpret_cast<const uint4*>(p.ab + row * w2 + col), a);
            unpack8(*reinterpret_cast<const uint4*>(p.ab + row * w2 + p.Nout + col), b);
            const float rs = p.row_scale[row];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float sg = 1.0f / (1.0f + expf(-a[e]));
              dot += dh[e] * (a[e] * sg * b[e]);
              const float d = rs * dh[e];
              da[e] = d * b[e] * sg * (1.0f + a[e] * (1.0f - sg));
              db[e] = d * a[e] * sg;
            }
            bf16_t* C = static_cast<bf16_t*>(p.C);
            *reinterpret_cast<uint4*>(C + row * w2 + col) = pack8(da);
            *reinterpret_cast<uint4*>(C + row * w2 + p.Nout + col) = pack8(db);
          }
          dot += __shfl_xor(dot, 1, 64);
          dot += __shfl_xor(dot, 2, 64);
          dot += __shfl_xor(dot, 4, 64);
          if (valid && c == 0)
            p.gate_part[row * (p.Nout / 64) + (t.nt * BN + wn * 64) / 64] = dot;
          continue;
        }
        if (!valid) continue;
        const u32x4_t vv = *(const LDS_AS u32x4_t*)(stg + stg_off(m, c));
        const uint4 v = make_uint4(vv.x, vv.y, vv.z, vv.w);
        const int64_t row = t.row0 + wm * 64 + ii * 32 + m;
        if (MODE == FWD || MODE == DGRAD) {
          bf16_t* C = static_cast<bf16_t*>(p.C);
          *reinterpret_cast<uint4*>(C + row * p.Nout + t.nt * BN + wn * 64 + 8 * c) = v;
        } else if (MODE == FWD_SWIGLU) {
          bf16_t* C = static_cast<bf16_t*>(p.C);
          const int64_t col = (c >> 2) * fh + t.nt * (BN / 2) + wn * 32 + (c & 3) * 8;
          *reinterpret_cast<uint4*>(C + row * p.Nout + col) = v;
        } else if (MODE == DGRAD_SWIGLU_BWD) {
          // v = dH[row, col .. col+7]; read the matching a and b, write dA and dB
          const int64_t col = t.nt * BN + wn * 64 + 8 * c;
          const int64_t w2 = 2 * p.Nout;
          float dh[8], a[8], b[8], da[8], db[8];
          unpack8(v, dh);
          unpack8(*reinterpret_cast<const uint4*>(p.ab + row * w2 + col), a);
          unpack8(*reinterpret_cast<const uint4*>(p.ab + row * w2 + p.Nout + col), b);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float sg = 1.0f / (1.0f + expf(-a[e]));
            da[e] = dh[e] * b[e] * sg * (1.0f + a[e] * (1.0f - sg));
            db[e] = dh[e] * a[e] * sg;
          }
          bf16_t* C = static_cast<bf16_t*>(p.C);
          *reinterpret_cast<uint4*>(C + row * w2 + col) = pack8(da);
          *reinterpret_cast<uint4*>(C + row * w2 + p.Nout + col) = pack8(db);
        } else {  // WGRAD, bf16 out
          bf16_t* C = static_cast<bf16_t*>(p.C) + static_cast<int64_t>(t.g) * p.Kc * p.Nout;
          uint4* q = reinterpret_cast<uint4*>(C + row * p.Nout + t.nt * BN + wn * 64 + 8 * c);
          if (p.accumulate) {
            float x[8], y[8];
            unpack8(v, x);
            unpack8(*q, y);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] += y[e];
            *q = pack8(x);
          } else {
            // streaming store: the gradient is not read again by this layer
            __builtin_nontemporal_store(vv, reinterpret_cast<u32x4_t*>(q));
          }
        }
      }
    }
    if (MODE == FWD_SWIGLU) {
      // H = silu(gate) * up (times the row's routing weight when it is
      // applied inside the expert) for these 32 rows: 32 columns per wave
      float rs = 1.0f;
      if (p.row_scale) {
        const int m = lane & 31;
        rs = ii * 32 + m < rows_w ? p.row_scale[t.row0 + wm * 64 + ii * 32 + m] : 0.0f;
      }
#pragma unroll
      for (int vg = 0; vg < 4; ++vg) {
        const int m = lane & 31;
        const int n = vg * 8 + (lane >> 5) * 4;
        float h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float g = acc[ii][0][vg * 4 + e], u = acc[ii][1][vg * 4 + e];
          h[e] = g / (1.0f + expf(-g)) * u * rs;
        }
        u32x2_t w;
        w.x = pack2(h[0], h[1]);
        w.y = pack2(h[2], h[3]);
        *(LDS_AS u32x2_t*)(stg + stg_off(m, n >> 3) + (n & 7) * 2) = w;
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int idx = lane + 64 * i;
        const int m = idx >> 2, c = idx & 3;
        if (ii * 32 + m >= rows_w) continue;
        const u32x4_t vv = *(const LDS_AS u32x4_t*)(stg + stg_off(m, c));
        const uint4 v = make_uint4(vv.x, vv.y, vv.z, vv.w);
        const int64_t row = t.row0 + wm * 64 + ii * 32 + m;
        *reinterpret_cast<uint4*>(p.H + row * fh + t.nt * (BN / 2) + wn * 32 + 8 * c) = v;
      }
    }
  }
}

// ---- the kernel ----------------------------------------------------------------

template <int MODE, int Q, int WN>
__global__ __launch_bounds__(Cfg<WN>::THREADS, Cfg<WN>::WG_PER_CU) void gg_kernel(Params p) {
  using C = Cfg<WN>;
  constexpr bool F8 = Q != P_BF16;
  constexpr int BN = C::BN;
  constexpr int NTH = C::THREADS;
  constexpr int SB = stage_bytes<WN, F8>();
  constexpr int PER = C::A_PER + C::B_PER + (F8 ? 1 : 0);  // DMA instructions per wave per stage
  __shared__ __attribute__((aligned(1024))) char ring[C::STAGES * SB];
  __shared__ int s_pre[MAX_GROUPS + 1];
  __shared__ int s_off[MAX_GROUPS + 1];  // row offsets (below 2^31)
  __shared__ int s_t256;                 // row tiles of the 256-row tiling
  LDS_AS char* lring = (LDS_AS char*)(ring);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // group offsets, clamped to a non-decreasing sequence in [0, M], kept in LDS
  // so that tile decoding never waits on vector memory
  for (int g = tid; g <= p.G; g += NTH) s_off[g] = static_cast<int>(clamp64(p.off[g], 0, p.M));
  __syncthreads();
  if (wave == 0) {  // running maximum makes the offsets non-decreasing
    const int per = (p.G + 1 + 63) / 64;
    const int g0 = lane * per, g1 = min(p.G + 1, g0 + per);
    int mx = 0;
    for (int g = g0; g < g1; ++g) mx = max(mx, s_off[g]);
    int incl = mx;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl = max(incl, y);
    }
    int run = __shfl_up(incl, 1, 64);
    if (lane == 0) run = 0;
    for (int g = g0; g < g1; ++g) {
      run = max(run, s_off[g]);
      s_off[g] = run;
    }
  }
  __syncthreads();

  int64_t NT, total;
  if (MODE == WGRAD) {
    NT = p.Nout / BN;
    total = static_cast<int64_t>(p.G) * (p.Kc / BM) * NT;
  } else {
    if (wave == 0) {
      const int per = (p.G + 63) / 64;
      const int g0 = lane * per, g1 = min(p.G, g0 + per);
      int sum = 0;
      for (int g = g0; g < g1; ++g) sum += (s_off[g + 1] - s_off[g] + BM - 1) / BM;
      int incl = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      int run = incl - sum;
      for (int g = g0; g < g1; ++g) {
        s_pre[g] = run;
        run += (s_off[g + 1] - s_off[g] + BM - 1) / BM;
      }
      if (lane == 63) s_pre[p.G] = incl;
      if (MODE != WGRAD) {
        int t256 = 0;
        for (int g = g0; g < g1; ++g) t256 += (s_off[g + 1] - s_off[g] + 255) / 256;
        t256 = wave_sum(t256);
        if (lane == 0) s_t256 = t256;
      }
    }
    __syncthreads();
    if (MODE != WGRAD && p.pair256 && rows256_preferred<MODE, Q>(s_pre[p.G], s_t256))
      return;  // the paired 256-row launch does the work
    NT = p.Nout / BN;
    total = static_cast<int64_t>(s_pre[p.G]) * NT;
  }

  const Walk walk = make_walk(total);
  int ld_i = 0, cp_i = 0;
  int64_t ld_tau = 0;
  Tile ld_t, cp_t;
  bool ld_ok = walk_next(walk, ld_i, total, ld_tau) &&
               decode<MODE, F8, BN>(ld_tau, p, s_pre, s_off, NT, total, ld_t);
  bool cp_ok = ld_ok;
  cp_t = ld_t;
  cp_i = ld_i;
  Loader<WN> L;
  if (ld_ok) setup_loader<MODE, Q, WN>(p, ld_t, wave, lane, L);
  int ld_kt = 0, cp_kt = 0;
  int inflight = 0, ld_slot = 0, cp_slot = 0;

  // prologue: STAGES - 1 steps in flight
  for (int s = 0; s < C::STAGES - 1 && ld_ok; ++s) {
    issue<F8, WN>(L, ld_kt, lring + ld_slot * SB, wave);
    ++inflight;
    ld_slot = ld_slot + 1 == C::STAGES ? 0 : ld_slot + 1;
    if (++ld_kt == ld_t.nk) {
      ld_kt = 0;
      ++ld_i;
      ld_ok = walk_next(walk, ld_i, total, ld_tau) &&
              decode<MODE, F8, BN>(ld_tau, p, s_pre, s_off, NT, total, ld_t);
      if (ld_ok) setup_loader<MODE, Q, WN>(p, ld_t, wave, lane, L);
    }
  }

  f32x16_t acc[2][2];
#pragma unroll
  for (int ii = 0; ii < 2; ++ii)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[ii][jj][v] = 0.f;

  while (cp_ok) {
    // this step's stage has landed in LDS for all waves (at most one younger
    // stage of this wave still outstanding)
    wait_barrier<PER>(inflight - 1);
    if (ld_ok) {  // refill the slot consumed in the previous step
      issue<F8, WN>(L, ld_kt, lring + ld_slot * SB, wave);
      ++inflight;
      ld_slot = ld_slot + 1 == C::STAGES ? 0 : ld_slot + 1;
      if (++ld_kt == ld_t.nk) {
        ld_kt = 0;
        ++ld_i;
        ld_ok = walk_next(walk, ld_i, total, ld_tau) &&
                decode<MODE, F8, BN>(ld_tau, p, s_pre, s_off, NT, total, ld_t);
        if (ld_ok) setup_loader<MODE, Q, WN>(p, ld_t, wave, lane, L);
      }
    }
    compute_stage<MODE, Q, WN>(acc, lring + cp_slot * SB, wm, wn, lane);
    --inflight;
    if (++cp_kt == cp_t.nk) {
      // the slot just consumed is not refilled before the next barrier: stage
      // there, once every wave has finished reading its fragments from it
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      // blockwise fp8 row groups otherwise spill inside the k loop
      epilogue<MODE, BN>(p, cp_t, acc, lring + cp_slot * SB + wave * 4096, wm, wn,
                         Q == P_FP8 && MODE != WGRAD ? opaque_lane() : lane);
#pragma unroll
      for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[ii][jj][v] = 0.f;
      cp_kt = 0;
      // the compute cursor follows the loader's walk one tile behind
      ++cp_i;
      int64_t cp_tau = 0;
      cp_ok = walk_next(walk, cp_i, total, cp_tau) &&
              decode<MODE, F8, BN>(cp_tau, p, s_pre, s_off, NT, total, cp_t);
    }
    cp_slot = cp_slot + 1 == C::STAGES ? 0 : cp_slot + 1;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int MODE, int Q, int WN>
static hipError_t run_cfg(const Params& p, int64_t tiles_upper_bound, hipStream_t s) {
  if (tiles_upper_bound <= 0) return hipSuccess;
  int64_t grid = static_cast<int64_t>(cu_count()) * Cfg<WN>::WG_PER_CU;  // persistent
  if (tiles_upper_bound < grid) grid = tiles_upper_bound;
  if (grid < 1) grid = 1;
  gg_kernel<MODE, Q, WN><<<dim3(static_cast<unsigned>(grid)), Cfg<WN>::THREADS, 0, s>>>(p);
  return hipGetLastError();
}

// bf16 row-group modes in 256 x 256 tiles (defined below); false when the
// shape does not fit them
template <int MODE, int Q>
static bool launch_rows256(const Params& p, hipStream_t s, hipError_t& err);

// Row-group modes: tiles of BM rows of a group x BN product columns (SwiGLU:
// BN/2 gate + BN/2 up columns); at most M/BM + G row tiles.  The wide tile
// whenever the product width allows it.
template <int MODE, int Q>
static hipError_t run_rows(const Params& p, hipStream_t s) {
  const int64_t mt = p.M / BM + p.G;
  if constexpr (Q != P_FP8) {
    // both tilings are launched; from the group sizes each kernel finds on
    // the device which of the two does the work, and the other one exits
    Params q = p;
    q.pair256 = 1;
    hipError_t err = hipSuccess;
    if (launch_rows256<MODE, Q>(q, s, err)) {
      if (err != hipSuccess) return err;
      return run_cfg<MODE, Q, 4>(q, mt * (p.Nout / 256), s);
    }
  }
  if (p.Nout % 256 == 0) return run_cfg<MODE, Q, 4>(p, mt * (p.Nout / 256), s);
  return run_cfg<MODE, Q, 2>(p, mt * (p.Nout / 128), s);
}

// ---- weight gradient, 256 x 256 tiles ---------------------------------------
// dB[g] = A[rows g]^T . dC[rows g] with both output dimensions multiples of
// 256 (no ragged output dimension, so the larger tile wastes nothing): 8 waves
// in a 4 x 2 arrangement, each 64 x 128 (2 x 4 MFMA 32x32 blocks), a 2-stage
// ring of 64 KiB operand stages.  bf16: A is 64 tokens x 256 columns, B the
// same, both in the [k][col] layout read with ds_read_b64_tr_b16.  MXFP8:
// the transposed token tiles, 256 rows x 128 tokens each in the [row][k]
// layout, plus one E8M0 dword per row and stage.  Against the
// 128 x 256 tile this halves the per-tile work of decoding, loader set-up and
// epilogue synchronisation per FLOP (a group's token range is short, so a
// tile is a few k steps), reads a quarter fewer LDS fragments per MFMA, and
// re-reads the activation slabs a quarter less.
namespace w256 {
constexpr int BMN = 256;           // tile rows (dB rows) and columns
constexpr int SLAB = 16384;        // bf16 [64 k][128 cols]; fp8 [128 rows][128 k]
constexpr int OPS = 4 * SLAB;      // A: 2 slabs, B: 2 slabs
constexpr int SCALES = 2048;       // fp8 / MX: 256 + 256 per-row scale words
template <int Q> constexpr int stage_bytes() { return OPS + (Q == P_BF16 ? 0 : SCALES); }
constexpr int STAGES = 2;
}

// [32 m][128 n] bf16 staging rows of 256 B, 16-byte chunks swizzled by m & 15
__device__ __forceinline__ int stg_off16(int m, int chunk) {
  return m * 256 + ((chunk ^ (m & 15)) << 4);
}

template <int Q>
__global__ __launch_bounds__(512, 1) void wgrad256_kernel(Params p) {
  using namespace w256;
  // blockwise fp8 keeps the 128-row tiles: its promotion of each partial by
  // two scales on the vector ALUs takes as long as the MFMAs in this tiling
  static_assert(Q != P_FP8, "bf16 and MXFP8 only");
  constexpr bool F8 = Q != P_BF16;
  constexpr int STAGE = stage_bytes<Q>();
  __shared__ __attribute__((aligned(1024))) char ring[STAGES * STAGE];
  __shared__ int s_off[MAX_GROUPS + 1];
  LDS_AS char* lring = (LDS_AS char*)(ring);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  for (int g = tid; g <= p.G; g += 512) s_off[g] = static_cast<int>(clamp64(p.off[g], 0, p.M));
  __syncthreads();
  if (wave == 0) {  // running maximum makes the offsets non-decreasing
    const int per = (p.G + 1 + 63) / 64;
    const int g0 = lane * per, g1 = min(p.G + 1, g0 + per);
    int mx = 0;
    for (int g = g0; g < g1; ++g) mx = max(mx, s_off[g]);
    int incl = mx;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl = max(incl, y);
    }
    int run = __shfl_up(incl, 1, 64);
    if (lane == 0) run = 0;
    for (int g = g0; g < g1; ++g) {
      run = max(run, s_off[g]);
      s_off[g] = run;
    }
  }
  __syncthreads();

  const uint32_t MT = static_cast<uint32_t>(p.Kc / BMN), NT = static_cast<uint32_t>(p.Nout / BMN);
  const uint32_t per_g = MT * NT;
  const int64_t total = static_cast<int64_t>(p.G) * per_g;
  const int64_t K = p.Kc, N = p.Nout;

  struct T256 {
    int g;
    int64_t row0, col0, lo, nrows;
    int nk;
  };
  auto decode256 = [&](int64_t tau, T256& t) {
    const uint32_t tu = static_cast<uint32_t>(tau);
    t.g = static_cast<int>(tu / per_g);
    uint32_t m, n;
    tile_in_group<WG_SN>(tu - static_cast<uint32_t>(t.g) * per_g, MT, NT, WG_SM, m, n);
    t.row0 = static_cast<int64_t>(m) * BMN;
    t.col0 = static_cast<int64_t>(n) * BMN;
    t.lo = s_off[t.g];
    t.nrows = s_off[t.g + 1] - t.lo;
    t.nk = t.nrows > 0 ? static_cast<int>((t.nrows + KStep<F8>::value - 1) / KStep<F8>::value) : 1;
  };
  // loader of a tile: DMA instruction q = wave * 4 + i of each operand fills
  // 1 KiB of slab q / 16 -- bf16: k rows 4 (q % 16) .. + 3 (256 bytes each);
  // MXFP8: rows 8 (q % 16) .. + 7 (128 bytes each) -- and, MXFP8, one E8M0
  // dword per row: waves 0-3 the 256 rows of A, waves 4-7 those of B
  i32x4_t ra, rb, rs;
  uint32_t va[4], vb[4], vs = 0, ds = 0;
  const int64_t ldm = p.ldm;
  auto setup = [&](const T256& t) {
    if (!F8) {
      ra = make_rsrc(p.A + t.lo * K * 2, static_cast<uint64_t>(t.nrows) * K * 2);
      rb = make_rsrc(p.B + t.lo * N * 2, static_cast<uint64_t>(t.nrows) * N * 2);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = wave * 4 + i, slab = q >> 4;
        const int kr = 4 * (q & 15) + (lane >> 4), c = (lane & 15) ^ swz_nc(kr);
        va[i] = static_cast<uint32_t>((kr * K + t.row0 + slab * 128 + 8 * c) * 2);
        vb[i] = static_cast<uint32_t>((kr * N + t.col0 + slab * 128 + 8 * c) * 2);
      }
      return;
    }
    // A = X^T codes [K, ldm], B = dC^T codes [N, ldm]: the tile's 256 rows,
    // contraction over the group's padded token range [lo, lo + nrows)
    const bool any = t.nrows > 0;
    ra = make_rsrc(p.A + t.row0 * ldm + t.lo, any ? static_cast<uint64_t>(BMN) * ldm : 0);
    rb = make_rsrc(p.B + t.col0 * ldm + t.lo, any ? static_cast<uint64_t>(BMN) * ldm : 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = wave * 4 + i, slab = q >> 4;
      const int r = 8 * (q & 15) + (lane >> 3), c = (lane & 7) ^ swz_kc(r);
      va[i] = static_cast<uint32_t>((slab * 128 + r) * ldm + c * 16);
      vb[i] = va[i];
    }
    const bool for_a = wave < 4;
    const int64_t row = (for_a ? t.row0 : t.col0) + (wave & 3) * 64 + lane;
    // E8M0 [K][ldm/32] / [N][ldm/32]: dword lo/128 + kt of each row
    rs = make_rsrc(for_a ? p.ea : p.eb, static_cast<uint64_t>(for_a ? K : N) * (ldm / 32));
    vs = static_cast<uint32_t>(row * (ldm / 32) + t.lo / 32);
    ds = 4;
  };
  const uint32_t da = F8 ? 128u : static_cast<uint32_t>(64 * K * 2);
  const uint32_t db = F8 ? 128u : static_cast<uint32_t>(64 * N * 2);
  auto issue = [&](int kt, LDS_AS char* stage) {
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(ra, stage + (wave * 4 + i) * 1024, va[i] + kt * da);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(rb, stage + 2 * SLAB + (wave * 4 + i) * 1024, vb[i] + kt * db);
    if (F8) dma4(rs, stage + OPS + wave * 256, vs + kt * ds);
  };

  const Walk walk = make_walk(total);
  int ld_i = 0, cp_i = 0;
  int64_t ld_tau = 0;
  T256 ld_t, cp_t;
  bool ld_ok = walk_next(walk, ld_i, total, ld_tau);
  if (ld_ok) {
    decode256(ld_tau, ld_t);
    setup(ld_t);
  }
  bool cp_ok = ld_ok;
  cp_t = ld_t;
  cp_i = ld_i;
  int ld_kt = 0, cp_kt = 0, ld_slot = 0, cp_slot = 0;
  auto advance_loader = [&]() {
    ld_slot ^= 1;
    if (++ld_kt == ld_t.nk) {
      ld_kt = 0;
      ++ld_i;
      ld_ok = walk_next(walk, ld_i, total, ld_tau);
      if (ld_ok) {
        decode256(ld_tau, ld_t);
        setup(ld_t);
      }
    }
  };
  if (ld_ok) {  // prologue: the first stage in flight
    issue(ld_kt, lring + ld_slot * STAGE);
    advance_loader();
  }

  f32x16_t acc[2][4];
#pragma unroll
  for (int ii = 0; ii < 2; ++ii)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[ii][jj][v] = 0.f;

  while (cp_ok) {
    // this step's stage has landed for every wave (nothing younger in flight)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (ld_ok) {  // the other slot was consumed before the barrier
      issue(ld_kt, lring + ld_slot * STAGE);
      advance_loader();
    }
    {
      const LDS_AS char* stage = lring + cp_slot * STAGE;
      const LDS_AS char* opA = stage + (wm >> 1) * SLAB;
      const LDS_AS char* opB = stage + 2 * SLAB + wn * SLAB;
      const int ra0 = (wm & 1) * 64;  // the wave's first row inside its A slab
      if (Q == P_BF16) {
        // tokens of the group left in this stage: a 16-token sub-step past
        // them holds only zero rows, so its MFMAs are skipped
        const int64_t left = cp_t.nrows - static_cast<int64_t>(cp_kt) * 64;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          if (kk * 16 >= left) break;
          bf16x8_t a[2], b[4];
#pragma unroll
          for (int ii = 0; ii < 2; ++ii) a[ii] = frag_nc(opA, ra0 + ii * 32, kk * 16, lane);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) b[jj] = frag_nc(opB, jj * 32, kk * 16, lane);
#pragma unroll
          for (int ii = 0; ii < 2; ++ii)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
              acc[ii][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[jj], a[ii], acc[ii][jj], 0, 0, 0);
        }
      } else if (Q == P_MX) {
        // scale words: A rows at 0.., B rows at 256..; see compute_stage_mx
        const LDS_AS uint32_t* eA = (const LDS_AS uint32_t*)(stage + OPS);
        const int h = lane >> 5;
        uint32_t xa[2], xb[4];
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) xa[ii] = eA[wm * 64 + ii * 32 + (lane & 31)] >> (8 * h);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) xb[jj] = eA[256 + wn * 128 + jj * 32 + (lane & 31)] >> (8 * h);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          i32x8_t a[2], b[4];
#pragma unroll
          for (int ii = 0; ii < 2; ++ii) a[ii] = frag_mx(opA, ra0 + ii * 32 + (lane & 31), s2, h);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) b[jj] = frag_mx(opB, jj * 32 + (lane & 31), s2, h);
#pragma unroll
          for (int ii = 0; ii < 2; ++ii)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
              acc[ii][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  b[jj], a[ii], acc[ii][jj], 0, 0, 0, static_cast<int>(xb[jj] >> (16 * s2)), 0,
                  static_cast<int>(xa[ii] >> (16 * s2)));
        }
      }
    }
    if (++cp_kt == cp_t.nk) {
      // the slot just consumed becomes the staging area once every wave has
      // read its fragments from it
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const int lane = Q == P_MX ? opaque_lane() : threadIdx.x & 63;  // MXFP8 spills otherwise
      const int64_t row_w = cp_t.row0 + wm * 64, col_w = cp_t.col0 + wn * 128;
      if (p.out_f32) {
        float* out = static_cast<float*>(p.C) + static_cast<int64_t>(cp_t.g) * K * N;
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int vg = 0; vg < 4; ++vg) {
              const int64_t m = row_w + ii * 32 + (lane & 31);
              const int64_t n = col_w + jj * 32 + vg * 8 + (lane >> 5) * 4;
              float4* q = reinterpret_cast<float4*>(out + m * N + n);
              float4 v = make_float4(acc[ii][jj][vg * 4], acc[ii][jj][vg * 4 + 1],
                                     acc[ii][jj][vg * 4 + 2], acc[ii][jj][vg * 4 + 3]);
              if (p.accumulate) {
                const float4 o = *q;
                v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
              }
              *q = v;
            }
      } else {
        LDS_AS char* stg = lring + cp_slot * STAGE + wave * 8192;
        bf16_t* out = static_cast<bf16_t*>(p.C) + static_cast<int64_t>(cp_t.g) * K * N;
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int vg = 0; vg < 4; ++vg) {
              const int m = lane & 31;
              const int n = jj * 32 + vg * 8 + (lane >> 5) * 4;
              u32x2_t w;
              w.x = pack2(acc[ii][jj][vg * 4 + 0], acc[ii][jj][vg * 4 + 1]);
              w.y = pack2(acc[ii][jj][vg * 4 + 2], acc[ii][jj][vg * 4 + 3]);
              *(LDS_AS u32x2_t*)(stg + stg_off16(m, n >> 3) + (n & 7) * 2) = w;
            }
          // 32 rows x 16 chunks; lane handles chunks lane + 64 i
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int idx = lane + 64 * i;
            const int m = idx >> 4, c = idx & 15;
            const u32x4_t vv = *(const LDS_AS u32x4_t*)(stg + stg_off16(m, c));
            uint4* q = reinterpret_cast<uint4*>(out + (row_w + ii * 32 + m) * N + col_w + 8 * c);
            if (p.accumulate) {
              float x[8], y[8];
              unpack8(make_uint4(vv.x, vv.y, vv.z, vv.w), x);
              unpack8(*q, y);
#pragma unroll
              for (int e = 0; e < 8; ++e) x[e] += y[e];
              *q = pack8(x);
            } else {
              // streaming store: the gradient is not read again by this layer
              __builtin_nontemporal_store(vv, reinterpret_cast<u32x4_t*>(q));
            }
          }
        }
      }
#pragma unroll
      for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[ii][jj][v] = 0.f;
      cp_kt = 0;
      ++cp_i;
      int64_t cp_tau = 0;
      cp_ok = walk_next(walk, cp_i, total, cp_tau);
      if (cp_ok) decode256(cp_tau, cp_t);
    }
    cp_slot ^= 1;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ---- bf16 row-group GEMMs (forward, dgrad), 256 x 256 tiles ------------------
// The forward (B = W_g [K, N] read in the [k][col] layout) and the data
// gradient (B = W_g [N, K] rows, k-contiguous) in tiles of 256 rows of a group
// x 256 product columns, waves and ring as in the weight-gradient kernel, with
// the same epilogues as the 128-row tiles: plain, SwiGLU (a tile holds 128
// gate columns and the matching 128 up columns, each wave 64 + 64 of them, so
// that H is formed in registers) and SwiGLU backward.  A group's last row tile
// is ragged (its rows past the group read as zero, so nothing is fetched for
// them); the larger tile halves the row tiles of a large group, hence its
// re-reads of the weight slabs, and moves a third fewer operand bytes per FLOP
// into LDS.
template <int MODE, int Q>
__global__ __launch_bounds__(512, 1) void rows256_kernel(Params p) {
  using namespace w256;
  constexpr bool MX = Q == P_MX;
  constexpr int STAGE = stage_bytes<Q>();
  constexpr bool B_NC = !MX && (MODE == FWD || MODE == FWD_SWIGLU);
  constexpr int ES = MX ? 1 : 2;  // operand element bytes
  __shared__ __attribute__((aligned(1024))) char ring[STAGES * STAGE];
  __shared__ int s_pre[MAX_GROUPS + 1];
  __shared__ int s_off[MAX_GROUPS + 1];
  __shared__ int s_t128;  // row tiles of the 128-row tiling
  LDS_AS char* lring = (LDS_AS char*)(ring);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  for (int g = tid; g <= p.G; g += 512) s_off[g] = static_cast<int>(clamp64(p.off[g], 0, p.M));
  __syncthreads();
  if (wave == 0) {  // running maximum makes the offsets non-decreasing
    const int per = (p.G + 1 + 63) / 64;
    const int g0 = lane * per, g1 = min(p.G + 1, g0 + per);
    int mx = 0;
    for (int g = g0; g < g1; ++g) mx = max(mx, s_off[g]);
    int incl = mx;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl = max(incl, y);
    }
    int run = __shfl_up(incl, 1, 64);
    if (lane == 0) run = 0;
    for (int g = g0; g < g1; ++g) {
      run = max(run, s_off[g]);
      s_off[g] = run;
    }
  }
  __syncthreads();
  if (wave == 0) {  // row-tile prefix of the groups
    const int per = (p.G + 63) / 64;
    const int g0 = lane * per, g1 = min(p.G, g0 + per);
    int sum = 0;
    for (int g = g0; g < g1; ++g) sum += (s_off[g + 1] - s_off[g] + BMN - 1) / BMN;
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    int run = incl - sum;
    for (int g = g0; g < g1; ++g) {
      s_pre[g] = run;
      run += (s_off[g + 1] - s_off[g] + BMN - 1) / BMN;
    }
    if (lane == 63) s_pre[p.G] = incl;
    int t128 = 0;
    for (int g = g0; g < g1; ++g) t128 += (s_off[g + 1] - s_off[g] + BM - 1) / BM;
    t128 = wave_sum(t128);
    if (lane == 0) s_t128 = t128;
  }
  __syncthreads();
  if (p.pair256 && !rows256_preferred<MODE, Q>(s_t128, s_pre[p.G])) return;  // the 128-row launch works

  const uint32_t NT = static_cast<uint32_t>(p.Nout / BMN);
  const int64_t total = static_cast<int64_t>(s_pre[p.G]) * NT;
  const int64_t Kc = p.Kc, N = p.Nout;
  const int nk = static_cast<int>(Kc / KStep<MX>::value);

  struct TR {
    int g;
    int64_t row0, col0;
    int rows;
  };
  auto decode = [&](int64_t tau64, TR& t) {
    const uint32_t tau = static_cast<uint32_t>(tau64);
    int glo = 0, ghi = p.G;
    while (ghi - glo > 1) {
      const int mid = (glo + ghi) >> 1;
      if (static_cast<uint32_t>(s_pre[mid]) * NT <= tau) glo = mid; else ghi = mid;
    }
    const int g = __builtin_amdgcn_readfirstlane(glo);
    t.g = g;
    const uint32_t base = static_cast<uint32_t>(s_pre[g]);
    const uint32_t mt_g = static_cast<uint32_t>(s_pre[g + 1]) - base;
    uint32_t m, n;
    tile_in_group<ROW_SN>(tau - base * NT, mt_g, NT, mt_g, m, n);
    const int64_t lo = s_off[g], hi = s_off[g + 1];
    t.row0 = lo + static_cast<int64_t>(m) * BMN;
    t.col0 = static_cast<int64_t>(n) * BMN;
    t.rows = static_cast<int>(min<int64_t>(BMN, hi - t.row0));
  };
  // MXFP8: B row (output column) of tile row rho; with SwiGLU slab s (one
  // wave column) holds gate columns col0 / 2 + 64 s .. + 63 in rows 0-63 and
  // the matching up columns in rows 64-127
  auto b_row_kc = [&](const TR& t, int rho) -> int64_t {
    if (MODE == FWD_SWIGLU)
      return ((rho & 127) >= 64 ? N / 2 : 0) + t.col0 / 2 + (rho >> 7) * 64 + (rho & 63);
    return t.col0 + rho;
  };
  i32x4_t ra, rb, rs;
  uint32_t va[4], vb[4], vs = 0;
  auto setup = [&](const TR& t) {
    ra = make_rsrc(p.A + t.row0 * Kc * ES, static_cast<uint64_t>(t.rows) * Kc * ES);
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // A: rows 8 (q % 16) .. + 7 of slab q / 16
      const int q = wave * 4 + i, slab = q >> 4;
      const int r = 8 * (q & 15) + (lane >> 3), c = (lane & 7) ^ swz_kc(r);
      va[i] = static_cast<uint32_t>((slab * 128 + r) * Kc * ES + c * 16);
    }
    if (B_NC) {  // W_g [Kc, N]: k rows 4 (q % 16) .. + 3, columns col0 + 128 slab ..
      rb = make_rsrc(p.B + static_cast<int64_t>(t.g) * Kc * N * 2, static_cast<uint64_t>(Kc) * N * 2);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = wave * 4 + i, slab = q >> 4;
        const int kr = 4 * (q & 15) + (lane >> 4), c = (lane & 15) ^ swz_nc(kr);
        // SwiGLU: tile n holds gate columns 128 n .. + 127 and the matching up
        // columns; slab s (one wave column) its gate columns 128 n + 64 s ..
        // + 63 as chunks 0-7 and the up columns as chunks 8-15
        const int64_t col = MODE == FWD_SWIGLU
                                ? (c >> 3) * (N / 2) + t.col0 / 2 + slab * 64 + (c & 7) * 8
                                : t.col0 + slab * 128 + 8 * c;
        vb[i] = static_cast<uint32_t>((kr * N + col) * 2);
      }
    } else {  // B rows k-contiguous: bf16 W_g [N, Kc]; MXFP8 W_g^T / W_g codes [N, Kc]
      rb = make_rsrc(p.B + static_cast<int64_t>(t.g) * N * Kc * ES,
                     static_cast<uint64_t>(N) * Kc * ES);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = wave * 4 + i, slab = q >> 4;
        const int r = 8 * (q & 15) + (lane >> 3), c = (lane & 7) ^ swz_kc(r);
        vb[i] = static_cast<uint32_t>(b_row_kc(t, slab * 128 + r) * Kc * ES + c * 16);
      }
    }
    if (MX) {
      // E8M0 bytes, one per 32 k: A [M][Kc/32] (rows past the group read as
      // zero), B [G][N][Kc/32]; dword kt of each row.  Waves 0-3 fetch the
      // 256 rows of A, waves 4-7 those of B.
      const int64_t nb = Kc / 32;
      if (wave < 4) {
        rs = make_rsrc(p.ea + t.row0 * nb, static_cast<uint64_t>(t.rows) * nb);
        vs = static_cast<uint32_t>((wave * 64 + lane) * nb);
      } else {
        rs = make_rsrc(p.eb + static_cast<int64_t>(t.g) * N * nb, static_cast<uint64_t>(N) * nb);
        vs = static_cast<uint32_t>(b_row_kc(t, (wave - 4) * 64 + lane) * nb);
      }
    }
  };
  const uint32_t da = 128u, db = B_NC ? static_cast<uint32_t>(64 * N * 2) : 128u;
  auto issue = [&](int kt, LDS_AS char* stage) {
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(ra, stage + (wave * 4 + i) * 1024, va[i] + kt * da);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(rb, stage + 2 * SLAB + (wave * 4 + i) * 1024, vb[i] + kt * db);
    if (MX) dma4(rs, stage + OPS + wave * 256, vs + kt * 4);
  };

  const Walk walk = make_walk(total);
  int ld_i = 0, cp_i = 0;
  int64_t ld_tau = 0;
  TR ld_t, cp_t;
  bool ld_ok = walk_next(walk, ld_i, total, ld_tau);
  if (ld_ok) {
    decode(ld_tau, ld_t);
    setup(ld_t);
  }
  bool cp_ok = ld_ok;
  cp_t = ld_t;
  cp_i = ld_i;
  int ld_kt = 0, cp_kt = 0, ld_slot = 0, cp_slot = 0;
  auto advance_loader = [&]() {
    ld_slot ^= 1;
    if (++ld_kt == nk) {
      ld_kt = 0;
      ++ld_i;
      ld_ok = walk_next(walk, ld_i, total, ld_tau);
      if (ld_ok) {
        decode(ld_tau, ld_t);
        setup(ld_t);
      }
    }
  };
  if (ld_ok) {
    issue(ld_kt, lring + ld_slot * STAGE);
    advance_loader();
  }

  f32x16_t acc[2][4];
#pragma unroll
  for (int ii = 0; ii < 2; ++ii)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[ii][jj][v] = 0.f;

  while (cp_ok) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (ld_ok) {
      issue(ld_kt, lring + ld_slot * STAGE);
      advance_loader();
    }
    if (cp_t.rows > wm * 64) {  // a wave whose 64 rows all lie past the group idles
      const LDS_AS char* stage = lring + cp_slot * STAGE;
      const LDS_AS char* opA = stage + (wm >> 1) * SLAB;
      const LDS_AS char* opB = stage + 2 * SLAB + wn * SLAB;
      const int ra0 = (wm & 1) * 64;
      if constexpr (MX) {
        // scale dwords: A rows at 0.., B rows at 256..; see compute_stage_mx
        const LDS_AS uint32_t* eA = (const LDS_AS uint32_t*)(stage + OPS);
        const int h = lane >> 5;
        uint32_t xa[2], xb[4];
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) xa[ii] = eA[wm * 64 + ii * 32 + (lane & 31)] >> (8 * h);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) xb[jj] = eA[256 + wn * 128 + jj * 32 + (lane & 31)] >> (8 * h);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          i32x8_t a[2], b[4];
#pragma unroll
          for (int ii = 0; ii < 2; ++ii) a[ii] = frag_mx(opA, ra0 + ii * 32 + (lane & 31), s2, h);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) b[jj] = frag_mx(opB, jj * 32 + (lane & 31), s2, h);
#pragma unroll
          for (int ii = 0; ii < 2; ++ii)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
              // format 0 = E4M3 for both; byte 0 of each scale operand is used
              acc[ii][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  b[jj], a[ii], acc[ii][jj], 0, 0, 0, static_cast<int>(xb[jj] >> (16 * s2)), 0,
                  static_cast<int>(xa[ii] >> (16 * s2)));
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          bf16x8_t a[2], b[4];
#pragma unroll
          for (int ii = 0; ii < 2; ++ii)
            a[ii] = frag_kc(opA, ra0 + ii * 32 + (lane & 31), kk * 2 + (lane >> 5));
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            b[jj] = B_NC ? frag_nc(opB, jj * 32, kk * 16, lane)
                         : frag_kc(opB, jj * 32 + (lane & 31), kk * 2 + (lane >> 5));
#pragma unroll
          for (int ii = 0; ii < 2; ++ii)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
              acc[ii][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[jj], a[ii], acc[ii][jj], 0, 0, 0);
        }
      }
    }
    if (++cp_kt == nk) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const int rows_w = cp_t.rows - wm * 64;  // valid rows of this wave
      if (rows_w > 0) {
        // MXFP8 and the SwiGLU forward spill inside the k loop otherwise
        const int lane = MX || MODE == FWD_SWIGLU ? opaque_lane() : threadIdx.x & 63;
        LDS_AS char* stg = lring + cp_slot * STAGE + wave * 8192;
        bf16_t* out = static_cast<bf16_t*>(p.C);
        const int64_t row_w = cp_t.row0 + wm * 64, col_w = cp_t.col0 + wn * 128;
        const int64_t fh = N / 2;
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
          if (ii * 32 >= rows_w) break;
          if (MODE != FWD_SWIGLU || out != nullptr) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
#pragma unroll
              for (int vg = 0; vg < 4; ++vg) {
                const int m = lane & 31;
                const int n = jj * 32 + vg * 8 + (lane >> 5) * 4;
                u32x2_t w;
                w.x = pack2(acc[ii][jj][vg * 4 + 0], acc[ii][jj][vg * 4 + 1]);
                w.y = pack2(acc[ii][jj][vg * 4 + 2], acc[ii][jj][vg * 4 + 3]);
                *(LDS_AS u32x2_t*)(stg + stg_off16(m, n >> 3) + (n & 7) * 2) = w;
              }
            // 32 rows x 16 chunks; lane handles chunks lane + 64 i
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const int idx = lane + 64 * i;
              const int m = idx >> 4, c = idx & 15;
              const bool valid = ii * 32 + m < rows_w;
              const int64_t row = row_w + ii * 32 + m;
              if (MODE == DGRAD_SWIGLU_BWD) {
                // v = dH[row, col .. col+7] (times the row's routing weight when
                // it is applied inside the expert); read the matching a and b,
                // write dA and dB, and with the weight the partial <dH', h> of
                // the row over each 64 columns (8 consecutive lanes hold them)
                const int64_t col = col_w + 8 * c;
                const int64_t w2 = 2 * N;
                float dot = 0.0f;
                if (valid) {
                  const u32x4_t vv = *(const LDS_AS u32x4_t*)(stg + stg_off16(m, c));
                  float dh[8], a[8], b[8], da[8], db[8];
                  unpack8(make_uint4(vv.x, vv.y, vv.z, vv.w), dh);
                  unpack8(*reinterpret_cast<const uint4*>(p.ab + row * w2 + col), a);
                  unpack8(*reinterpret_cast<const uint4*>(p.ab + row * w2 + N + col), b);
                  const float rs = p.row_scale ? p.row_scale[row] : 1.0f;
#pragma unroll
                  for (int e = 0; e < 8; ++e) {
                    const float sg = 1.0f / (1.0f + expf(-a[e]));
                    dot += dh[e] * (a[e] * sg * b[e]);
                    const float d = rs * dh[e];
                    da[e] = d * b[e] * sg * (1.0f + a[e] * (1.0f - sg));
                    db[e] = d * a[e] * sg;
                  }
                  *reinterpret_cast<uint4*>(out + row * w2 + col) = pack8(da);
                  *reinterpret_cast<uint4*>(out + row * w2 + N + col) = pack8(db);
                }
                if (p.row_scale) {
                  dot += __shfl_xor(dot, 1, 64);
                  dot += __shfl_xor(dot, 2, 64);
                  dot += __shfl_xor(dot, 4, 64);
                  if (valid && (c & 7) == 0) p.gate_part[row * (N / 64) + col / 64] = dot;
                }
                continue;
              }
              if (!valid) continue;
              const u32x4_t vv = *(const LDS_AS u32x4_t*)(stg + stg_off16(m, c));
              const int64_t col = MODE == FWD_SWIGLU
                                      ? (c >> 3) * fh + cp_t.col0 / 2 + wn * 64 + (c & 7) * 8
                                      : col_w + 8 * c;
              *reinterpret_cast<u32x4_t*>(out + row * N + col) = vv;
            }
          }
          if (MODE == FWD_SWIGLU) {
            // H = silu(gate) * up (times the row's routing weight when it is
            // applied inside the expert) for these 32 rows: blocks jj and
            // jj + 2 hold matching gate and up columns, 64 per wave
            float rs = 1.0f;
            if (p.row_scale) {
              const int m = lane & 31;
              rs = ii * 32 + m < rows_w ? p.row_scale[row_w + ii * 32 + m] : 0.0f;
            }
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
              for (int vg = 0; vg < 4; ++vg) {
                const int m = lane & 31;
                const int n = jj * 32 + vg * 8 + (lane >> 5) * 4;
                float h[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const float g = acc[ii][jj][vg * 4 + e], u = acc[ii][jj + 2][vg * 4 + e];
                  h[e] = g / (1.0f + expf(-g)) * u * rs;
                }
                u32x2_t w;
                w.x = pack2(h[0], h[1]);
                w.y = pack2(h[2], h[3]);
                *(LDS_AS u32x2_t*)(stg + stg_off16(m, n >> 3) + (n & 7) * 2) = w;
              }
            // 32 rows x 8 chunks
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int idx = lane + 64 * i;
              const int m = idx >> 3, c = idx & 7;
              if (ii * 32 + m >= rows_w) continue;
              const u32x4_t vv = *(const LDS_AS u32x4_t*)(stg + stg_off16(m, c));
              *reinterpret_cast<u32x4_t*>(p.H + (row_w + ii * 32 + m) * fh + cp_t.col0 / 2 + wn * 64 +
                                          8 * c) = vv;
            }
          }
        }
      }
#pragma unroll
      for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[ii][jj][v] = 0.f;
      cp_kt = 0;
      ++cp_i;
      int64_t cp_tau = 0;
      cp_ok = walk_next(walk, cp_i, total, cp_tau);
      if (cp_ok) decode(cp_tau, cp_t);
    }
    cp_slot ^= 1;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int MODE, int Q>
static bool launch_rows256(const Params& p, hipStream_t s, hipError_t& err) {
  constexpr int BK = KStep<Q != P_BF16>::value;
  if (p.Nout % w256::BMN != 0 || p.Kc % BK != 0 || p.Kc < BK || !p.pair256) return false;
  const int64_t tiles = (p.M / w256::BMN + p.G) * (p.Nout / w256::BMN);
  int64_t grid = cu_count();  // persistent, one workgroup per CU
  if (tiles < grid) grid = tiles;
  if (grid < 1) grid = 1;
  rows256_kernel<MODE, Q><<<dim3(static_cast<unsigned>(grid)), 512, 0, s>>>(p);
  err = hipGetLastError();
  return true;
}

template <int Q>
static hipError_t run_wgrad(const Params& p, hipStream_t s) {
  // (blockwise fp8 keeps the 128-row tiles: in the 256 x 256 tiling its
  // promotion of each partial on the vector ALUs takes as long as the MFMAs,
  // and the weight gradients measured 1.4 times slower)
  if (Q != P_FP8 && p.Kc % w256::BMN == 0 && p.Nout % w256::BMN == 0) {
    const int64_t tiles = static_cast<int64_t>(p.G) * (p.Kc / w256::BMN) * (p.Nout / w256::BMN);
    if (tiles <= 0) return hipSuccess;
    int64_t grid = cu_count();  // persistent, one workgroup per CU
    if (tiles < grid) grid = tiles;
    wgrad256_kernel<Q == P_MX ? P_MX : P_BF16><<<dim3(static_cast<unsigned>(grid)), 512, 0, s>>>(p);
    return hipGetLastError();
  }
  const int64_t mt = static_cast<int64_t>(p.G) * (p.Kc / BM);
  if (p.Nout % 256 == 0) return run_cfg<WGRAD, Q, 4>(p, mt * (p.Nout / 256), s);
  return run_cfg<WGRAD, Q, 2>(p, mt * (p.Nout / 128), s);
}

static Params make_params(const void* A, const void* B, const int64_t* off, int G, int64_t M,
                          int64_t Kc, int64_t Nout, void* C, void* H, const void* ab) {
  Params p{};
  p.A = static_cast<const char*>(A);
  p.B = static_cast<const char*>(B);
  p.off = off;
  p.G = G;
  p.M = M;
  p.Kc = Kc;
  p.Nout = Nout;
  p.C = C;
  p.H = static_cast<bf16_t*>(H);
  p.ab = static_cast<const bf16_t*>(ab);
  return p;
}

hipError_t launch_gg_bf16_fwd(const void* A, const void* B, const int64_t* off, int G, int64_t M,
                              int64_t K, int64_t N, int epi, void* C, void* H, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const Params p = make_params(A, B, off, G, M, K, N, C, H, nullptr);
  if (epi == EPI_SWIGLU) return run_rows<FWD_SWIGLU, P_BF16>(p, s);
  return run_rows<FWD, P_BF16>(p, s);
}

hipError_t launch_gg_bf16_dgrad(const void* dC, const void* B, const int64_t* off, int G,
                                int64_t M, int64_t K, int64_t N, int epi, const void* ab, void* dA,
                                hipStream_t s) {
  if (M == 0) return hipSuccess;
  // contraction over N, product columns K
  const Params p = make_params(dC, B, off, G, M, N, K, dA, nullptr, ab);
  if (epi == EPI_SWIGLU_BWD) return run_rows<DGRAD_SWIGLU_BWD, P_BF16>(p, s);
  return run_rows<DGRAD, P_BF16>(p, s);
}

hipError_t launch_gg_bf16_wgrad(const void* A, const void* dC, const int64_t* off, int G,
                                int64_t M, int64_t K, int64_t N, int db_f32, int accumulate,
                                void* dB, hipStream_t s) {
  Params p = make_params(A, dC, off, G, M, K, N, dB, nullptr, nullptr);
  p.out_f32 = db_f32;
  p.accumulate = accumulate;
  return run_wgrad<P_BF16>(p, s);
}

hipError_t launch_gg_bf16_gated_fwd(const void* A, const void* B, const int64_t* off, int G,
                                    int64_t M, int64_t K, int64_t N, const float* row_scale,
                                    void* AB, void* H, hipStream_t s) {
  if (M == 0) return hipSuccess;
  Params p = make_params(A, B, off, G, M, K, N, AB, H, nullptr);
  p.row_scale = row_scale;
  return run_rows<FWD_SWIGLU, P_BF16>(p, s);
}

hipError_t launch_gg_bf16_gated_dgrad(const void* dC, const void* B, const int64_t* off, int G,
                                      int64_t M, int64_t K, int64_t N, const void* ab,
                                      const float* row_scale, void* dAB, float* gate_part,
                                      hipStream_t s) {
  if (M == 0) return hipSuccess;
  Params p = make_params(dC, B, off, G, M, N, K, dAB, nullptr, ab);
  p.row_scale = row_scale;
  p.gate_part = gate_part;
  return run_rows<DGRAD_SWIGLU_BWD, P_BF16>(p, s);
}

hipError_t launch_gg_fp8_fwd(const uint8_t* A, const float* sa, const uint8_t* Bt, const float* sb,
                             const int64_t* off, int G, int64_t M, int64_t K, int64_t N, int epi,
                             void* C, void* H, hipStream_t s) {
  if (M == 0) return hipSuccess;
  Params p = make_params(A, Bt, off, G, M, K, N, C, H, nullptr);
  p.sa = sa;
  p.sb = sb;
  if (epi == EPI_SWIGLU) return run_rows<FWD_SWIGLU, P_FP8>(p, s);
  return run_rows<FWD, P_FP8>(p, s);
}

hipError_t launch_gg_fp8_dgrad(const uint8_t* dC, const float* sa, const uint8_t* B,
                               const float* sb, const int64_t* off, int G, int64_t M, int64_t K,
                               int64_t N, int epi, const void* ab, void* dA, hipStream_t s) {
  if (M == 0) return hipSuccess;
  Params p = make_params(dC, B, off, G, M, N, K, dA, nullptr, ab);
  p.sa = sa;
  p.sb = sb;
  if (epi == EPI_SWIGLU_BWD) return run_rows<DGRAD_SWIGLU_BWD, P_FP8>(p, s);
  return run_rows<DGRAD, P_FP8>(p, s);
}

hipError_t launch_gg_fp8_wgrad(const uint8_t* At, const float* sa, const uint8_t* dCt,
                               const float* sb, const int64_t* poff, int G, int64_t ldm, int64_t K,
                               int64_t N, int db_f32, int accumulate, void* dB, hipStream_t s) {
  Params p = make_params(At, dCt, poff, G, ldm, K, N, dB, nullptr, nullptr);
  p.sa = sa;
  p.sb = sb;
  p.ldm = ldm;
  p.out_f32 = db_f32;
  p.accumulate = accumulate;
  return run_wgrad<P_FP8>(p, s);
}

hipError_t launch_gg_mx_fwd(const uint8_t* A, const uint8_t* ea, const uint8_t* Bt,
                            const uint8_t* eb, const int64_t* off, int G, int64_t M, int64_t K,
                            int64_t N, int epi, void* C, void* H, hipStream_t s) {
  if (M == 0) return hipSuccess;
  Params p = make_params(A, Bt, off, G, M, K, N, C, H, nullptr);
  p.ea = ea;
  p.eb = eb;
  if (epi == EPI_SWIGLU) return run_rows<FWD_SWIGLU, P_MX>(p, s);
  return run_rows<FWD, P_MX>(p, s);
}

hipError_t launch_gg_mx_dgrad(const uint8_t* dC, const uint8_t* ea, const uint8_t* B,
                              const uint8_t* eb, const int64_t* off, int G, int64_t M, int64_t K,
                              int64_t N, int epi, const void* ab, void* dA, hipStream_t s) {
  if (M == 0) return hipSuccess;
  Params p = make_params(dC, B, off, G, M, N, K, dA, nullptr, ab);
  p.ea = ea;
  p.eb = eb;
  if (epi == EPI_SWIGLU_BWD) return run_rows<DGRAD_SWIGLU_BWD, P_MX>(p, s);
  return run_rows<DGRAD, P_MX>(p, s);
}

hipError_t launch_gg_mx_wgrad(const uint8_t* At, const uint8_t* ea, const uint8_t* dCt,
                              const uint8_t* eb, const int64_t* poff, int G, int64_t ldm, int64_t K,
                              int64_t N, int db_f32, int accumulate, void* dB, hipStream_t s) {
  Params p = make_params(At, dCt, poff, G, ldm, K, N, dB, nullptr, nullptr);
  p.ea = ea;
  p.eb = eb;
  p.ldm = ldm;
  p.out_f32 = db_f32;
  p.accumulate = accumulate;
  return run_wgrad<P_MX>(p, s);
}

}  // namespace moe
