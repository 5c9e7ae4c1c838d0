// Grouped GEMMs of the expert SwiGLU FFN, forward and backward, on gfx950 MFMA.
//
// The expert FFN (SwiGLU with intermediate size F: the --ffn_dim of the
// Triton-distributed ep_moe_fused benchmark page) runs as one grouped GEMM per
// projection over the expert-sorted rows built by dispatch.  Six GEMM kinds:
//
//   mode               C (M x N)            A (M x K)             B (N x K)
//   GATE_UP_FWD        [G|U] rows x F       expand_x  (K-contig)  Wg_e, Wu_e (K-contig)
//   DOWN_FWD           y rows x H           h_act     (K-contig)  Wd_e       (K-contig)
//   DOWN_BWD_DATA      dH rows x F          grad_y    (K-contig)  Wd_e       (N-contig)
//   GATE_UP_BWD_DATA   dX rows x H          grad_gu   (K-contig)  [Wg_e;Wu_e](N-contig)
//   DOWN_BWD_W         dWd_e H x F          grad_y    (M-contig)  h_act      (N-contig)
//   GATE_UP_BWD_W      [dWg_e;dWu_e] 2F x H grad_gu   (M-contig)  expand_x   (N-contig)
//
// The first four are grouped over M (each expert owns a contiguous row range of
// the expanded buffers); the last two are grouped over K (the contraction runs
// over the expert's rows, which may be none).
//
// Operand types: bf16; fp8 e4m3 with fp32 scales (activations per (row, 128 of
// K), weights per 128 x 128 block; weight gradients per (128 tokens, column));
// microscaled e4m3 (MX: E8M0 scale per 32 of K, applied by the MFMA); int8 (one
// scale per row and per output channel; forward GEMMs only).
//
// Tiling: a BM x BN output tile per workgroup of WM x WN waves (128 x 128 or
// 128 x 256 with 2 x 2 waves, 256 x 256 with 2 x 4 waves, per GEMM kind and
// shape, see launch()), each wave (BM/WM) x (BN/WN) of
// v_mfma_f32_32x32x16_bf16 tiles (fp8: v_mfma_scale_f32_32x32x64_f8f6f4, with
// unit scales and the fp32 scales applied per 128-wide K block, or with the MX
// scales; int8: v_mfma_i32_32x32x32_i8), one to three workgroups per CU.  K
// steps of 64 or 32 (8-bit: 128 codes) go from memory straight into LDS
// (buffer loads with an LDS destination, no register staging), two or three
// LDS stages: the loads of the next steps are in flight while the MFMAs of
// step t issue.
// Operands keep their memory layout in LDS:
// K-contiguous tiles as rows of 2 BK bytes with an XOR-swizzled chunk order
// (one conflict-free 16-byte read per MFMA operand), K-strided tiles as
// k-rows read into MFMA operands with the transposing LDS read.  Every mode
// accumulates transposed fragments, so each lane holds runs of four output
// columns for the epilogue.
//
// Expert counts stay on the device: the grid covers floor(capacity/BM) + E row
// tiles per column tile, and each workgroup finds its expert from the prefix
// counts with one wave ballot (expert e owns row-tile slots starting at
// prefix[e-1]/BM + e); surplus workgroups exit at once.  Workgroups are dealt
// to the XCDs so that neighbouring tiles share an L2 (row-grouped modes, in
// groups of row tiles when the output is wide) and every XCD gets a block of
// every expert (weight gradients).
#include "common.hpp"

namespace moe {
namespace {

enum Mode : int {
  GATE_UP_FWD = 0,
  DOWN_FWD = 1,
  DOWN_BWD_DATA = 2,
  GATE_UP_BWD_DATA = 3,
  DOWN_BWD_W = 4,
  GATE_UP_BWD_W = 5
};

// The K step of the bf16 GEMMs (BK elements, 64 or 32) is a parameter of the
// kernel; the fp8 GEMMs step by 128 codes, one 128-byte LDS row, like a
// 64-element bf16 step.
// fp8 GEMMs: at most this many 128-wide K blocks (K <= 32768)
constexpr int kMaxKBlocks8 = 256;
// compute units of an MI355X (gfx950): 8 XCDs of 32
constexpr int kCUs = 256;
// gfx9 s_waitcnt immediate that waits for at most n outstanding vector memory
// operations (vmcnt in bits 3:0 and 15:14) and leaves the other counters free
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
// buffer resource word 3 for raw (untyped, unswizzled) buffer loads on gfx9:
// 32-bit data format, so every access is checked against the byte range only
constexpr int kBufferFlags = 0x00020000;

struct GemmArgs {
  const bf16_t* A;
  int64_t lda;
  // bf16 gate/up forward only: when set, A is the token matrix x and row r of
  // the expert-sorted operand is x[gather[r] / gK] (gather = the row -> slot
  // map of the routing, gK = top-K), so the dispatch permute is not needed
  const int32_t* gather;
  int gK;
  int64_t gbytes;  // bytes of x (T * H * 2): the range of the gathered loads
  // down data and weight gradients with the A operand gathered from grad_out:
  // row r of the expert-sorted grad_y is rowsc[r] * grad_out[slot(r) / K],
  // rowsc[r] the routing weight of the row's slot; the weight gradient forms it
  // as the combine backward stores it, bf16(rowsc[r] * grad_out), the data
  // gradient multiplies each row's fp32 product with W_down by rowsc[r]
  const float* rowsc;
  // gate/up weight gradient with the B operand gathered (rows of x read through
  // the row -> slot map): rows of the map (capacity), and slot / K as
  // (slot * kmagic) >> kshift (exact for slots below 2^31)
  int64_t grows;
  uint64_t kmagic;
  int kshift;
  const bf16_t* B0;
  const bf16_t* B1;
  int64_t ldb;
  int64_t bstride;  // elements between consecutive experts' B0/B1 matrices
  const int32_t* prefix;
  int E;
  int64_t M, N, Kd, F;
  int64_t n_tiles, m_tiles, tiles;
  int64_t mch, nch;  // weight gradients: tiles per block along M and N
  int kp;            // weight gradients: row blocks of an expert's tile grid
  int64_t gm;        // row-grouped GEMMs: row tiles per rasterisation group
  int krot;          // K steps of stagger between tiles sharing an operand tile
  bf16_t* C0;
  bf16_t* C1;
  const bf16_t* aux;
  float* W0;
  float* W1;
  // fp8 operands: e4m3 codes, A scales per (row, 128 of K) stored K-block major
  // (sA[kblock * rowsA + row], so a K step's scales of consecutive rows are
  // consecutive), B scales per 128 x 128 block at sB[e*sbe + nblock*sbn + kblock*sbk]
  const uint8_t* qA;
  const float* sA;
  const uint8_t* qB0;
  const uint8_t* qB1;
  const float* sB0;
  const float* sB1;
  int64_t sbe, sbn, sbk;
  int64_t rowsA;  // rows of the expanded activations (capacity)
  // fp8 down data gradient: optional e4m3 codes of the bf16 dG/dU it produces,
  // per (row, 128 columns) (qr/sr, the layout of moe_quant_rows_fp8) and per
  // (128-token slot, column) (qc/sc, the layout of moe_quant_cols_fp8, ldq
  // codes per row)
  uint8_t* qr;
  float* sr;
  uint8_t* qc;
  float* sc;
  int64_t ldq;
  // microscaled fp8 (MX): E8M0 scale bytes, one per 32 codes along K, stored as
  // one 4-byte word per (row, 128-code K step), words ordered (K step, row): A
  // has mrA rows per K step; B (weights) mrB rows per K step, mbe per expert
  // (gate/up data gradient: mB0 for K < F, mB1 for the rest)
  const uint8_t* mA;
  const uint8_t* mB0;
  const uint8_t* mB1;
  int64_t mrA, mrB, mbe;
  // MX forward / down data gradient: optional MX row codes of the bf16 output
  // (h, or dG|dU), in the layout of the MX row quantiser over rowsA rows
  uint8_t* qmx;
  uint8_t* smx;
};

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

// bf16(w[i] * v[i]) of the eight bf16 values of a fragment: one fp32 product and
// one round to nearest even each, the arithmetic of the combine backward's grad_y
// rows (for finite values the hardware conversion rounds as the written-out one does)
__device__ __forceinline__ bf16x8 scale_bf16x8_each(bf16x8 v, const float* w) {
  float f[8];
  unpack8(__builtin_bit_cast(uint4, v), f);
  const uint4 o = make_uint4(pk_bf16(w[0] * f[0], w[1] * f[1]), pk_bf16(w[2] * f[2], w[3] * f[3]),
                             pk_bf16(w[4] * f[4], w[5] * f[5]), pk_bf16(w[6] * f[6], w[7] * f[7]));
  return __builtin_bit_cast(bf16x8, o);
}

// LDS operand tile: R rows x W k of bf16, row pitch 2W bytes, in 16-byte
// chunks of 8 consecutive k.  Chunk c of row r sits at chunk position
// c ^ swz(r).  The LDS serves 256 bytes (64 banks of 4 bytes) per cycle, so
// the 16 lanes of one 16-byte read phase (16 consecutive rows, one chunk
// each) must cover the 16 distinct 16-byte slots of a 256-byte window:
// W = 64 (128-byte rows, two rows per window) swizzles by (r ^ r/8) % 8;
// W = 32 (64-byte rows, four rows per window) by (r/4) % 4.
template <int W>
__device__ __forceinline__ int swzw(int r) {
  if constexpr (W == 64) return (r ^ (r >> 3)) & 7;
  else return (r >> 2) & 3;
}
template <int W>
__device__ __forceinline__ int lds_offw(int r, int c) { return r * W + ((c ^ swzw<W>(r)) << 3); }

constexpr int cmax(int a, int b) { return a > b ? a : b; }
// weight gradients: fp32 output staged through LDS for full-line stores
constexpr bool kStagedWgrad = true;

// Compile-time shape of one kernel instance: BM x BN output tile.
template <int MODE, int BM, int BN, bool FP8, int BK, int S_, int WM_ = 2, int WN_ = 2>
struct Cfg {
  static_assert(BK == 64 || BK == 32, "K step of 32 or 64 bf16");
  static_assert(BM >= 128 && BN >= 128, "K-strided tiles swizzle over 16 chunks of a k-row");
  static constexpr bool KGROUP = MODE == DOWN_BWD_W || MODE == GATE_UP_BWD_W;
  static constexpr bool B_KC = MODE == GATE_UP_FWD || MODE == DOWN_FWD;
  // WM x WN waves, each a (BM/WM) x (BN/WN) block of TI x TJ MFMA 32x32 tiles
  static constexpr int WM = WM_, WN = WN_, kThreads = 64 * WM * WN;
  static constexpr int TI = BM / WM / 32, TJ = BN / WN / 32;
  // output columns staged in LDS at once by the epilogue, and its row pitch
  // (16 bytes of padding per row)
  static constexpr int CW = MODE == GATE_UP_FWD ? BN / 2 : BN;
  static constexpr int CP = CW + 8;
  // LDS stages of the bf16 operand tiles (the 8-bit paths have two)
  static constexpr int S = S_;
  // bf16: S stages of BK-wide tiles; 8-bit: two stages of 128-byte rows
  static constexpr int kMain = FP8 ? 2 * (BM + BN) * 64 : S * (BM + BN) * BK;
  // epilogue staging: h, G and U side by side when the three fit the operand
  // LDS, else h and G, then U (two passes) or one after the other (three);
  // the SwiGLU backward stages the saved G and U tiles, per wave column when
  // the whole tile does not fit the operand LDS (the fp8 down data gradient
  // stages them in one pass even beyond its operand LDS, at two workgroups
  // per CU: measured 5% faster than per wave column)
  static constexpr bool kEpiOnePass =
      MODE == GATE_UP_FWD ? 3 * BM * CP <= kMain
                          : (MODE == DOWN_BWD_DATA ? (FP8 ? 2 * BM * CP * 2 <= 80 * 1024 : 2 * BM * CP <= kMain) : true);
  static constexpr int CPH = BN / WN + 8;  // pitch of one wave column's staging
  // gate/up forward beyond the operand LDS: h and G in one pass, then U
  static constexpr bool kEpiGU2 = MODE == GATE_UP_FWD && !kEpiOnePass && 2 * BM * CP * 2 <= 160 * 1024;
  // (weight gradients: half the fp32 tile, 16 bytes of padding per row)
  static constexpr int kEpi =
      KGROUP ? (BM / 2) * (BN + 4) * 2
             : (MODE == GATE_UP_FWD ? (kEpiOnePass ? 3 : (kEpiGU2 ? 2 : 1)) * BM * CP
                                    : (MODE == DOWN_BWD_DATA ? (kEpiOnePass ? 2 * BM * CP : 2 * BM * CPH) : BM * CP));
  static constexpr int kSmem = cmax(kMain, kEpi);
  // workgroups per CU that the LDS allows (160 KB per CU), at most three
  static constexpr int kMinBlocks =
      kSmem * 2 <= 160 * 1024 / 3 ? 3 : (kSmem * 2 <= 80 * 1024 ? 2 : 1);
};

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// I8 (with FP8 set: the 8-bit operand path): int8 codes with one scale per A
// row and one per B row (output channel), integer MFMAs accumulated over the
// whole K, the scales applied once after the loop.
// MX (with FP8 set): e4m3 codes with E8M0 scales per 32 codes along K, applied by
// the MFMA itself (no per-step rescale).
template <int MODE, int BM, int BN, bool FP8, int BK, int S_, int WM_, int WN_, bool I8, bool MX>
__global__ __launch_bounds__((Cfg<MODE, BM, BN, FP8, BK, S_, WM_, WN_>::kThreads),
                             (Cfg<MODE, BM, BN, FP8, BK, S_, WM_, WN_>::kMinBlocks)) void k_gemm(GemmArgs g) {
  using C = Cfg<MODE, BM, BN, FP8, BK, S_, WM_, WN_>;
  static_assert(!I8 || (FP8 && (MODE == GATE_UP_FWD || MODE == DOWN_FWD)), "int8: forward GEMMs on the 8-bit path");
  static_assert(!MX || (FP8 && !I8 && MODE <= GATE_UP_BWD_DATA), "MX: row-grouped GEMMs on the 8-bit path");
  auto swz = [](int r) { return swzw<BK>(r); };
  auto lds_off = [](int r, int c) { return lds_offw<BK>(r, c); };
  constexpr bool KGROUP = C::KGROUP, B_KC = C::B_KC;
  constexpr int TI = C::TI, TJ = C::TJ;
  // S LDS stages of the A and B tiles; after the K loop the same memory
  // stages the output tile (and, for the SwiGLU backward, the saved G/U tile).
  __shared__ __attribute__((aligned(16))) bf16_t smem[C::kSmem];
  // fp8 operand stages: BM (BN) rows of 128 bytes, two stages
  auto As = [&](int st) { return smem + st * BM * 64; };
  auto Bs = [&](int st) { return smem + 2 * BM * 64 + st * BN * 64; };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int WM = C::WM, WN = C::WN, kThreads = C::kThreads;
  static_assert(!FP8 || kThreads == 256 || MX || I8, "the fp32-scaled fp8 loop is written for four waves");
  const int wm = wave / WN, wn = wave % WN;

  const int64_t nb = gridDim.x;
  const int64_t bid = blockIdx.x;
  // Workgroups are dispatched round-robin over the eight XCDs (XCD = bid % 8).
  // Row-grouped GEMMs: XCD x takes the x-th contiguous eighth of the tiles;
  // the work per row tile is the same for every expert, so the eighths are
  // balanced, and neighbouring tiles (same A rows, same expert weights) share
  // an L2.  Expert-grouped (weight-gradient) GEMMs: a tile's work grows with
  // its expert's row count, so each expert's tile grid is cut into eight
  // blocks (kp row blocks x 8/kp column blocks) and every XCD takes one block
  // of every expert (block (x + e) % 8), which balances any routing skew; an
  // XCD then reads 1/kp of the expert's A column strips and kp/8 of its B
  // strips (A is read 8/kp times over the chip and B kp times, instead of
  // eight times each).
  int e;
  int64_t row0, n0, kbeg, kend;
  int rows_valid;
  int kseed = 0;  // (row tile + column tile) % 8: staggers the K start, see krot
  int64_t tile_m = 0;  // row tile (row-grouped GEMMs): with BM = 128, the rows' token slot
  if constexpr (!KGROUP) {
    const int64_t logical = (bid & 7) * (nb >> 3) + (bid >> 3);
    if (logical >= g.tiles) return;
    // within an XCD's eighth, tiles go in groups of gm row tiles, column tile
    // by column tile: the workgroups in flight on one XCD then cover about
    // gm row tiles x (their number / gm) column tiles, so an expert's weight
    // tiles are fetched into L2 once per gm row tiles instead of once per row
    // tile when the layer is wide (gm = 1: row tile by row tile)
    const int64_t gsz = g.gm * g.n_tiles;
    const int64_t grp = logical / gsz, rem = logical - grp * gsz;
    const int64_t first = grp * g.gm;
    const int64_t gm = (g.m_tiles - first) < g.gm ? (g.m_tiles - first) : g.gm;
    const int64_t mt = first + rem % gm;
    const int64_t nt = rem / gm;
    kseed = (int)((mt + nt) & 7);
    tile_m = mt;
    // the expert index is the same in every lane; readfirstlane keeps it (and
    // every address derived from it) in scalar registers
    e = __builtin_amdgcn_readfirstlane(find_expert<BM>(g.prefix, g.E, mt));
    const int64_t p0 = e ? g.prefix[e - 1] : 0, p1 = g.prefix[e];
    row0 = p0 + (mt - (p0 / BM + e)) * BM;
    if (row0 >= p1) return;
    rows_valid = (int)((p1 - row0) < BM ? (p1 - row0) : BM);
    n0 = nt * (MODE == GATE_UP_FWD ? BN / 2 : BN);
    kbeg = 0;
    kend = g.Kd;
  } else {
    const int64_t xcd = bid & 7, k = bid >> 3;
    const int64_t per = g.mch * g.nch;  // tiles of one block
    e = (int)(k / per);
    if (e >= g.E) return;
    const int64_t w = k % per;
    const int blk = (int)((xcd + e) & 7);
    const int kq = 8 / g.kp;
    // within the block, groups of eight row tiles, column tile by column tile
    // (the same grouped order as the wide row-grouped GEMMs)
    constexpr int64_t kGroup = 8;
    const int64_t gsz = kGroup * g.nch;
    const int64_t grp = w / gsz, rem = w - grp * gsz;
    const int64_t first = grp * kGroup;
    const int64_t gmm = (g.mch - first) < kGroup ? (g.mch - first) : kGroup;
    const int64_t mt = (blk / kq) * g.mch + first + rem % gmm;
    const int64_t nt = (blk % kq) * g.nch + rem / gmm;
    if (mt >= g.m_tiles || nt >= g.n_tiles) return;
    row0 = mt * BM;  // first output row (weight row)
    n0 = nt * BN;
    kbeg = e ? g.prefix[e - 1] : 0;
    kend = g.prefix[e];
    rows_valid = (int)((g.M - row0) < BM ? (g.M - row0) : BM);
  }
  const int64_t klen = kend - kbeg;

  f32x16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  // B-tile row of MFMA column tile j of this wave.  The gate/up forward tile
  // holds BN/2 gate rows then the same BN/2 up rows, and each wave takes
  // matching gate and up column tiles so SwiGLU pairs meet in one lane.
  auto brow = [&](int j) -> int {
    if constexpr (MODE == GATE_UP_FWD)
      return (j < TJ / 2) ? wn * (BN / 2 / WN) + j * 32 : BN / 2 + wn * (BN / 2 / WN) + (j - TJ / 2) * 32;
    else
      return wn * (BN / WN) + j * 32;
  };
  int arow[TI], brw[TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i) arow[i] = wm * (BM / WM) + i * 32 + (lane & 31);
#pragma unroll
  for (int j = 0; j < TJ; ++j) brw[j] = brow(j) + (lane & 31);

  if constexpr (FP8) {
  // fp8 path: e4m3 codes, K-contiguous for both operands, K a multiple of 128.
  // One K step is 128 codes = one 128-byte LDS row per operand row, loaded
  // straight into LDS like the bf16 K-contiguous tiles (same swizzle, two
  // stages); two 32x32x64 MFMA sub-steps go into a temporary, then
  // acc += tmp * (A row scale * B block scale).  The accumulators hold
  // transposed fragments, so a lane's values share one row (one A scale) and
  // one j tile (one B block scale).  Weight gradients (KGROUP): both operands
  // are per-128-token codes, transposed (one row per output row or column,
  // the expert's token slots along it), a K step is one slot, and its scales
  // are one per A row and one per B column: acc += tmp * (A scale * B scale)
  // element by element.  MX: the MFMA applies the E8M0 scales, straight into
  // the accumulators; int8: integer MFMAs, scales applied after the loop.
  constexpr int S8 = 2;
  constexpr int LA = BM / 8 / (WM * WN), LB = BN / 8 / (WM * WN);
  static_assert(C::kMain >= S8 * (BM + BN) * 64, "fp8 stages must fit the operand LDS");
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  auto rsrc8 = [](const void* p) -> i32x4 {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                 __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xffff), 0x7ffffff0, kBufferFlags};
  };
  auto dma8 = [](const i32x4& r, const bf16_t* lds, uint32_t vo) {
    const uint32_t m0 = (uint32_t)reinterpret_cast<uintptr_t>(
        (const __attribute__((address_space(3))) bf16_t*)(lds));
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(vo), "s"(r), "{m0}"(m0));
  };
  uint32_t voA[LA], voB[LB];
#pragma unroll
  for (int j = 0; j < LA; ++j) {
    const int r = 8 * (wave * LA + j) + (lane >> 3), c = (lane & 7) ^ swzw<64>(r);
    const int rr = r < rows_valid ? r : rows_valid - 1;
    voA[j] = (uint32_t)(rr * g.lda + c * 16);
  }
#pragma unroll
  for (int j = 0; j < LB; ++j) {
    const int r = 8 * (wave * LB + j) + (lane >> 3), c = (lane & 7) ^ swzw<64>(r);
    int64_t n;
    if constexpr (MODE == GATE_UP_FWD) {
      n = n0 + (r & (BN / 2 - 1));
      if (n >= g.F) n = g.F - 1;
    } else {
      n = n0 + r;
      if (n >= g.N) n = g.N - 1;
    }
    voB[j] = (uint32_t)(n * g.ldb + c * 16);
  }
  const uint8_t* qa = g.qA + row0 * g.lda;
  // weight gradients: the expert's first token slot (K step 0)
  const int64_t slot0 = KGROUP ? kbeg / 128 + e : 0;
  // B codes of K step k0 (gate/up forward: half 1 = the up matrix; gate/up
  // data gradient: the gate codes for k < F, the up codes after)
  auto bsrc = [&](int64_t k0, int half) -> const uint8_t* {
    if constexpr (MODE == GATE_UP_FWD) {
      return (half ? g.qB1 : g.qB0) + (int64_t)e * g.bstride + k0;
    } else if constexpr (KGROUP) {
      return g.qB0 + k0;
    } else if constexpr (MODE == GATE_UP_BWD_DATA) {
      return k0 < g.F ? g.qB0 + (int64_t)e * g.bstride + k0 : g.qB1 + (int64_t)e * g.bstride + (k0 - g.F);
    } else {
      return g.qB0 + (int64_t)e * g.bstride + k0;
    }
  };
  auto bscale = [&](int64_t k0, int half) -> float {
    const int64_t kb = k0 / 128;
    if constexpr (MODE == GATE_UP_FWD) {
      const float* sb = half ? g.sB1 : g.sB0;
      return sb[e * g.sbe + (n0 / 128) * g.sbn + kb * g.sbk];
    } else if constexpr (MODE == GATE_UP_BWD_DATA) {
      const int64_t fb = g.F / 128;
      return kb < fb ? g.sB0[e * g.sbe + (n0 / 128) * g.sbn + kb * g.sbk]
                     : g.sB1[e * g.sbe + (n0 / 128) * g.sbn + (kb - fb) * g.sbk];
    } else {
      return g.sB0[e * g.sbe + (n0 / 128) * g.sbn + kb * g.sbk];
    }
  };
  auto issue8 = [&](auto ST, int64_t kt) {
    constexpr int st = decltype(ST)::value;
    const int64_t k0 = (slot0 + kt) * 128;
    const auto ra = rsrc8(qa + k0);
#pragma unroll
    for (int j = 0; j < LA; ++j) dma8(ra, As(st) + (wv * LA + j) * 512, voA[j]);
    const auto rb0 = rsrc8(bsrc(k0, 0));
    const auto rb1 = rsrc8(bsrc(k0, 1));
#pragma unroll
    for (int j = 0; j < LB; ++j) {
      const int q = wv * LB + j;
      const bool up = MODE == GATE_UP_FWD && 8 * q >= BN / 2;
      dma8(up ? rb1 : rb0, Bs(st) + q * 512, voB[j]);
    }
  };
  // A row scales of step kt go to LDS with the tiles (one 4-byte load per
  // tile row, issued by wave 0): a plain vector load here would make the
  // compiler wait for every load in flight, the tile loads included
  // (weight gradients: the B column scales of step kt go the same way, into
  // sBl[st][0, BN))
  __shared__ float sAl[2][BM];
  __shared__ float sBl[2][kMaxKBlocks8];
  static_assert(!KGROUP || BN <= kMaxKBlocks8, "B column scales of one step fit sBl");
  uint32_t vos[BM / 64], vosb[BN / 64];
#pragma unroll
  for (int q = 0; q < BM / 64; ++q) {
    const int r = q * 64 + lane;
    const int rr = r < rows_valid ? r : rows_valid - 1;
    vos[q] = (uint32_t)(rr * 4);
  }
#pragma unroll
  for (int q = 0; q < BN / 64; ++q) {
    if constexpr (MX) {
      // B tile row q*64 + lane: its channel relative to n0 (gate/up forward: rows
      // BN/2.. are the up matrix's channels n0..)
      const int rb = MODE == GATE_UP_FWD ? ((q * 64 + lane) & (BN / 2 - 1)) : q * 64 + lane;
      const int64_t lim = (MODE == GATE_UP_FWD ? g.F : g.N) - 1 - n0;
      vosb[q] = (uint32_t)((rb < lim ? rb : lim) * 4);
    } else {
      const int64_t n = n0 + q * 64 + lane;
      vosb[q] = (uint32_t)(((n < g.N ? n : g.N - 1) - n0) * 4);
    }
  }
  auto lds_dword = [](const i32x4& r, const float* lds, uint32_t vo) {
    const uint32_t m0 = (uint32_t)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) float*)(lds));
    asm volatile("buffer_load_dword %0, %1, 0 offen lds" : : "v"(vo), "s"(r), "{m0}"(m0));
  };
  auto issue_scales = [&](auto ST, int64_t kt) {
    constexpr int st = decltype(ST)::value;
    if (wv != 0) return;
    if constexpr (MX) {
      // the step's four scale bytes of each A row and each B row, one dword each
      const auto ra = rsrc8(g.mA + (kt * g.mrA + row0) * 4);
#pragma unroll
      for (int q = 0; q < BM / 64; ++q) lds_dword(ra, &sAl[st][q * 64], vos[q]);
#pragma unroll
      for (int q = 0; q < BN / 64; ++q) {
        const uint8_t* base;
        if constexpr (MODE == GATE_UP_FWD)
          base = (q * 64 >= BN / 2 ? g.mB1 : g.mB0) + (kt * g.mrB + e * g.mbe + n0) * 4;
        else if constexpr (MODE == GATE_UP_BWD_DATA)
          base = kt * 128 < g.F ? g.mB0 + (kt * g.mrB + e * g.mbe + n0) * 4
                                : g.mB1 + ((kt - g.F / 128) * g.mrB + e * g.mbe + n0) * 4;
        else
          base = g.mB0 + (kt * g.mrB + e * g.mbe + n0) * 4;
        lds_dword(rsrc8(base), &sBl[st][q * 64], vosb[q]);
      }
    } else if constexpr (KGROUP) {
      const auto ra = rsrc8(g.sA + (slot0 + kt) * g.M + row0);
#pragma unroll
      for (int q = 0; q < BM / 64; ++q) lds_dword(ra, &sAl[st][q * 64], vos[q]);
      const auto rb = rsrc8(g.sB0 + (slot0 + kt) * g.N + n0);
#pragma unroll
      for (int q = 0; q < BN / 64; ++q) lds_dword(rb, &sBl[st][q * 64], vosb[q]);
    } else {
      const auto r = rsrc8(g.sA + kt * g.rowsA + row0);
#pragma unroll
      for (int q = 0; q < BM / 64; ++q) lds_dword(r, &sAl[st][q * 64], vos[q]);
    }
  };
  auto compute8 = [&](auto ST, int64_t kt) {
    constexpr int st = decltype(ST)::value;
    const bf16_t* as = As(st);
    const bf16_t* bs = Bs(st);
    if constexpr (MX) {
      // two 32x32x64 MFMAs per 128-code step, the E8M0 scales applied by the
      // MFMA: its K block 0 is bytes 0-15 of lanes 0-31 then of lanes 32-63
      // (scale from lanes 0-31), block 1 their bytes 16-31 (scale from lanes
      // 32-63), so lane l takes chunks 4 kk + l/32 and 4 kk + 2 + l/32 and the
      // two blocks are the step's 32-code blocks 2 kk and 2 kk + 1; the row's
      // four scale bytes, shifted by one byte in lanes 32-63, give both blocks'
      // scales at byte 2 kk
      uint32_t sar[TI], sbr[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) sar[i] = __float_as_uint(sAl[st][arow[i]]) >> (8 * (lane >> 5));
#pragma unroll
      for (int j = 0; j < TJ; ++j) sbr[j] = __float_as_uint(sBl[st][brw[j]]) >> (8 * (lane >> 5));
      auto sub = [&](auto KK) {
        constexpr int kk = decltype(KK)::value;
        const int clo = 4 * kk + (lane >> 5), chi = clo + 2;
        i32x8 fa[TI], fb[TJ];
#pragma unroll
        for (int i = 0; i < TI; ++i) {
          const uint4 lo = *reinterpret_cast<const uint4*>(as + lds_offw<64>(arow[i], clo));
          const uint4 hi = *reinterpret_cast<const uint4*>(as + lds_offw<64>(arow[i], chi));
          fa[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const uint4 lo = *reinterpret_cast<const uint4*>(bs + lds_offw<64>(brw[j], clo));
          const uint4 hi = *reinterpret_cast<const uint4*>(bs + lds_offw<64>(brw[j], chi));
          fb[j] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j], fa[i], acc[i][j], 0, 0, 2 * kk,
                                                                       (int)sbr[j], 2 * kk, (int)sar[i]);
      };
      sub(std::integral_constant<int, 0>());
      sub(std::integral_constant<int, 1>());
      return;
    } else if constexpr (I8) {
      // four 32x32x32 int8 MFMAs per 128-code step; lane l supplies the 16
      // codes of chunk 2 kk + l/32 of its row (the same K split for A and B,
      // which is all a dot product needs)
      typedef int i32x16 __attribute__((ext_vector_type(16)));
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int c = kk * 2 + (lane >> 5);
        i32x4 fa[TI], fb[TJ];
#pragma unroll
        for (int i = 0; i < TI; ++i) fa[i] = *reinterpret_cast<const i32x4*>(as + lds_offw<64>(arow[i], c));
#pragma unroll
        for (int j = 0; j < TJ; ++j) fb[j] = *reinterpret_cast<const i32x4*>(bs + lds_offw<64>(brw[j], c));
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j)
            acc[i][j] = __builtin_bit_cast(
                f32x16, __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[j], fa[i], __builtin_bit_cast(i32x16, acc[i][j]), 0, 0, 0));
      }
      return;
    } else {
    f32x16 tmp[TI][TJ];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c = kk * 4 + (lane >> 5) * 2;
      i32x8 fa[TI], fb[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const uint4 lo = *reinterpret_cast<const uint4*>(as + lds_offw<64>(arow[i], c));
        const uint4 hi = *reinterpret_cast<const uint4*>(as + lds_offw<64>(arow[i], c + 1));
        fa[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const uint4 lo = *reinterpret_cast<const uint4*>(bs + lds_offw<64>(brw[j], c));
        const uint4 hi = *reinterpret_cast<const uint4*>(bs + lds_offw<64>(brw[j], c + 1));
        fb[j] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          if (kk == 0) {
            f32x16 z;
#pragma unroll
            for (int r = 0; r < 16; ++r) z[r] = 0.f;
            // e4m3 x e4m3 (format 0 for both), unit E8M0 scales (127)
            tmp[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j], fa[i], z, 0, 0, 0, 127, 0, 127);
          } else {
            tmp[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j], fa[i], tmp[i][j], 0, 0, 0,
                                                                         127, 0, 127);
          }
        }
    }
    if constexpr (KGROUP) {
      // column n = brow(j) + 8 t + 4 (lane/32) + q of the tile: runs of four
      // consecutive B scales
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        float4 sb[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
          sb[t] = *reinterpret_cast<const float4*>(&sBl[st][brow(j) + 8 * t + 4 * (lane >> 5)]);
#pragma unroll
        for (int i = 0; i < TI; ++i) {
          const float sa = sAl[st][wm * (BM / WM) + i * 32 + (lane & 31)];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            acc[i][j][4 * t + 0] += tmp[i][j][4 * t + 0] * (sa * sb[t].x);
            acc[i][j][4 * t + 1] += tmp[i][j][4 * t + 1] * (sa * sb[t].y);
            acc[i][j][4 * t + 2] += tmp[i][j][4 * t + 2] * (sa * sb[t].z);
            acc[i][j][4 * t + 3] += tmp[i][j][4 * t + 3] * (sa * sb[t].w);
          }
        }
      }
    } else {
      float sbv[TJ];
#pragma unroll
      for (int j = 0; j < TJ; ++j) sbv[j] = sBl[(MODE == GATE_UP_FWD && j >= TJ / 2) ? 1 : 0][kt];
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const float f = sAl[st][wm * (BM / WM) + i * 32 + (lane & 31)] * sbv[j];
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] += tmp[i][j][r] * f;
        }
    }
    }
  };
  // K steps: 128-wide blocks of K, or the expert's token slots
  const int64_t nk = KGROUP ? (klen + 127) / 128 : g.Kd / 128;
  // B block scales of every K step, read once before the pipeline starts
  if constexpr (!KGROUP && !I8 && !MX)
    for (int64_t kb = tid; kb < nk; kb += kThreads) {
      sBl[0][kb] = bscale(kb * 128, 0);
      if (MODE == GATE_UP_FWD) sBl[1][kb] = bscale(kb * 128, 1);
    }
  auto kstep8 = [&](auto ST, int64_t kt) {
    constexpr int st = decltype(ST)::value;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kt + 1 < nk) {
      issue8(std::integral_constant<int, st ^ 1>(), kt + 1);
      if constexpr (!I8) issue_scales(std::integral_constant<int, st ^ 1>(), kt + 1);
    }
    compute8(ST, kt);
  };
  if (nk > 0) {
    issue8(std::integral_constant<int, 0>(), 0);
    if constexpr (!I8) issue_scales(std::integral_constant<int, 0>(), 0);
  }
  for (int64_t kt = 0; kt < nk; kt += 2) {
    kstep8(std::integral_constant<int, 0>(), kt);
    if (kt + 1 < nk) kstep8(std::integral_constant<int, 1>(), kt + 1);
  }
  __syncthreads();
  if constexpr (I8) {
    // integer sums times (A row scale x B channel scale): B tile row rb is
    // channel n0 + rb (gate/up: rows BN/2.. are the up matrix's channels
    // n0 + rb - BN/2); a lane's four consecutive rows rb share a float4 of scales
    typedef int i32x16 __attribute__((ext_vector_type(16)));
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int m = wm * (BM / WM) + i * 32 + (lane & 31);
      const float sa = g.sA[row0 + (m < rows_valid ? m : rows_valid - 1)];
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const i32x16 ai = __builtin_bit_cast(i32x16, acc[i][j]);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int rb = brow(j) + 8 * t + 4 * (lane >> 5);
          float4 sb;
          if constexpr (MODE == GATE_UP_FWD)
            sb = *reinterpret_cast<const float4*>((rb >= BN / 2 ? g.sB1 : g.sB0) + (int64_t)e * g.F + n0 +
                                                  (rb & (BN / 2 - 1)));
          else
            sb = *reinterpret_cast<const float4*>(g.sB0 + (int64_t)e * g.N + n0 + rb);
          acc[i][j][4 * t + 0] = (float)ai[4 * t + 0] * (sa * sb.x);
          acc[i][j][4 * t + 1] = (float)ai[4 * t + 1] * (sa * sb.y);
          acc[i][j][4 * t + 2] = (float)ai[4 * t + 2] * (sa * sb.z);
          acc[i][j][4 * t + 3] = (float)ai[4 * t + 3] * (sa * sb.w);
        }
      }
    }
  }
  } else {
  // Operand tiles go from memory straight into LDS (buffer loads with an LDS
  // destination: lane l of one instruction writes the 16 bytes at
  // instruction base + 16 l), in the operand's own memory layout:
  //  * K-contiguous operand of R rows: R rows x 2 BK bytes, chunk c of row r
  //    at chunk position c ^ swz(r); one instruction fills 512/BK rows, lane l
  //    taking row (512/BK) q + l/(BK/8), position l%(BK/8), i.e. memory chunk
  //    position ^ swz(row).
  //  * K-strided operand of R columns: BK k-rows x 2R bytes, 16-byte chunk c
  //    of k-row k at position c ^ (4 (k%4)); one instruction fills 512/R
  //    k-rows.  MFMA fragments come out of it with transposing LDS reads
  //    (ds_read_b64_tr_b16: within each 16-lane group, lane i receives
  //    element i of the group's four 8-byte rows read in lane order, for
  //    each of the four rows), two reads per 8-k fragment.  The 32 lanes of
  //    one read phase take four chunks of four k-rows; the swizzle puts them
  //    in the 16 distinct 16-byte slots of a 256-byte bank window.
  // Rows past the operand are clamped to its last row (their products only
  // reach output rows or columns that are not stored).  Past the end of the
  // contraction the loads return zero: K-strided operands through the range
  // of the buffer resource (its byte count ends at the last k-row), the
  // K-contiguous A through an out-of-range offset in the last step.
  constexpr int S = C::S;
  // load instructions per wave per stage (an R x BK tile is R*BK/512
  // instructions of 1 KB)
  constexpr int LA = BM * BK / 512 / (WM * WN), LB = BN * BK / 512 / (WM * WN);
  constexpr int CPRK = BK / 8, RPIK = 64 / CPRK;  // K-contiguous: chunks per row, rows per instruction
  constexpr uint32_t kOOB = 0x80000000u;
  constexpr int kRange = 0x7ffffff0;
  auto sw4 = [](int k) { return 4 * (k & 3); };
  // buffer resource (base, byte range) in scalar registers
  auto rsrc = [](const void* p, int64_t bytes) -> i32x4 {
    const int64_t n = bytes < 0 ? 0 : (bytes < kRange ? bytes : kRange);
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                 __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xffff),
                 __builtin_amdgcn_readfirstlane((int)n), kBufferFlags};
  };
  // One 16-byte-per-lane load into LDS at byte address `lds` (+ 16 * lane).
  // Written as an instruction of its own so that the compiler, which would
  // otherwise wait for every such load before any LDS read, leaves the
  // waiting to the pipeline below (explicit vmcnt waits); the instruction has
  // no register result.
  auto dma = [](const i32x4& r, const bf16_t* lds, uint32_t vo) {
    const uint32_t m0 = (uint32_t)reinterpret_cast<uintptr_t>(
        (const __attribute__((address_space(3))) bf16_t*)(lds));
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(vo), "s"(r), "{m0}"(m0));
  };
  // per-lane byte offsets of this wave's load instructions (relative to the
  // step's base) and the K offset of the lane's chunk (K-contiguous operands)
  uint32_t voA[LA], voB[LB];
  int kcA[LA], kcB[LB];
#pragma unroll
  for (int j = 0; j < LA; ++j) {
    const int q = wave * LA + j;
    if constexpr (!KGROUP) {
      const int r = RPIK * q + lane / CPRK, c = (lane % CPRK) ^ swz(r);
      const int rr = r < rows_valid ? r : rows_valid - 1;
      int64_t arow = rr;  // row of A relative to abase
      if constexpr ((MODE == GATE_UP_FWD || MODE == DOWN_BWD_DATA) && !FP8)
        if (g.gather) arow = g.gather[row0 + rr] / g.gK;  // the token of this expanded row
      voA[j] = (uint32_t)((arow * g.lda + c * 8) * 2);
      kcA[j] = c * 8;
    } else {
      constexpr int CPR = BM / 8, RPI = 64 / CPR;
      const int k = RPI * q + lane / CPR, c = (lane % CPR) ^ sw4(k);
      const int64_t col = row0 + c * 8 < g.M ? row0 + c * 8 : g.M - 8;
      voA[j] = (uint32_t)((k * g.lda + col) * 2);
      kcA[j] = 0;
    }
  }
#pragma unroll
  for (int j = 0; j < LB; ++j) {
    const int q = wave * LB + j;
    if constexpr (B_KC) {
      const int r = RPIK * q + lane / CPRK, c = (lane % CPRK) ^ swz(r);
      int64_t n;
      if constexpr (MODE == GATE_UP_FWD) {
        n = n0 + (r & (BN / 2 - 1));
        if (n >= g.F) n = g.F - 1;
      } else {
        n = n0 + r;
        if (n >= g.N) n = g.N - 1;
      }
      voB[j] = (uint32_t)((n * g.ldb + c * 8) * 2);
      kcB[j] = c * 8;
    } else {
      constexpr int CPR = BN / 8, RPI = 64 / CPR;
      const int k = RPI * q + lane / CPR, c = (lane % CPR) ^ sw4(k);
      const int64_t col = n0 + c * 8 < g.N ? n0 + c * 8 : g.N - 8;
      voB[j] = (uint32_t)((k * g.ldb + col) * 2);
      kcB[j] = 0;
    }
  }
  const bool gathered = (MODE == GATE_UP_FWD || MODE == DOWN_BWD_DATA) && !FP8 && g.gather;
  // gate/up weight gradient reading the rows of x through the row -> slot map:
  // lane k-rows and byte columns of its B loads, and a ring of the map's entries
  // per K step (8 steps of 64), filled by wave 0 with direct-to-LDS loads two
  // steps ahead of the step whose tile loads need them
  constexpr bool GATHER_B = MODE == GATE_UP_BWD_W && !FP8;
  const bool gatherB = GATHER_B && g.gather;
  // down weight gradient reading grad_out rows through the same map (A operand),
  // each k-row scaled by its routing weight: the weights of a K step's k-rows go
  // into LDS with the step's tiles (wave 0, one dword per lane)
  constexpr bool GATHER_A = MODE == DOWN_BWD_W && !FP8;
  const bool gatherA = GATHER_A && g.gather;
  __shared__ int32_t tokr[(GATHER_A || GATHER_B) ? 8 * 64 : 1];
  __shared__ __attribute__((aligned(16))) float wst[GATHER_A ? S * 64 : 1];
  int kA[LA];
  uint32_t colA[LA];
  if constexpr (GATHER_A) {
#pragma unroll
    for (int j = 0; j < LA; ++j) {
      constexpr int CPR = BM / 8, RPI = 64 / CPR;
      const int q = wave * LA + j;
      const int k = RPI * q + lane / CPR, c = (lane % CPR) ^ sw4(k);
      kA[j] = k;
      colA[j] = (uint32_t)((row0 + c * 8 < g.M ? row0 + c * 8 : g.M - 8) * 2);
    }
  }
  int kB[LB];
  uint32_t colB[LB];
#pragma unroll
  for (int j = 0; j < LB; ++j) {
    constexpr int CPR = BN / 8, RPI = 64 / CPR;
    const int q = wave * LB + j;
    const int k = RPI * q + lane / CPR, c = (lane % CPR) ^ sw4(k);
    kB[j] = k;
    colB[j] = (uint32_t)((n0 + c * 8 < g.N ? n0 + c * 8 : g.N - 8) * 2);
  }
  const char* abase =
      reinterpret_cast<const char*>(KGROUP ? g.A + kbeg * g.lda : (gathered ? g.A : g.A + row0 * g.lda));
  const char* bbase0;
  const char* bbase1;
  if constexpr (KGROUP) {
    bbase0 = bbase1 = reinterpret_cast<const char*>(g.B0 + kbeg * g.ldb);
  } else {
    bbase0 = reinterpret_cast<const char*>(g.B0 + (int64_t)e * g.bstride);
    bbase1 = reinterpret_cast<const char*>((MODE == GATE_UP_FWD || MODE == GATE_UP_BWD_DATA)
                                               ? g.B1 + (int64_t)e * g.bstride
                                               : g.B0 + (int64_t)e * g.bstride);
  }
  const int wv = __builtin_amdgcn_readfirstlane(wave);  // wave index, in a scalar register

  // direct loads of K step kt into LDS stage ST
  auto issue = [&](auto ST, int64_t kt) {
    constexpr int st = decltype(ST)::value;
    const int64_t k0 = kt * BK;
    const bool tail = k0 + BK > klen;
    bf16_t* sa = smem + st * BM * BK;
    bf16_t* sb = smem + S * BM * BK + st * BN * BK;
    if constexpr (!KGROUP) {
      // gathered rows: the range ends at the end of x, so a token offset from
      // a stale or foreign row -> slot map reads zeros instead of past x
      const auto r = rsrc(abase + k0 * 2, gathered ? g.gbytes - k0 * 2 : kRange);
#pragma unroll
      for (int j = 0; j < LA; ++j) {
        const uint32_t vo = (tail && k0 + kcA[j] >= kend) ? kOOB : voA[j];
        dma(r, sa + (wv * LA + j) * 512, vo);
      }
    } else if (GATHER_A && gatherA) {
      // k-row k of the step is expanded row kbeg + k0 + k: grad_out row slot/K;
      // k-rows past the expert's end read zeros
      const auto r = rsrc(g.A, g.gbytes);
      const int32_t* tk = tokr + (kt & 7) * 64;
#pragma unroll
      for (int j = 0; j < LA; ++j) {
        uint32_t vo = kOOB;
        if (k0 + kA[j] < klen) {
          const uint32_t sl = (uint32_t)tk[kA[j]];
          const uint32_t tok = (uint32_t)(((uint64_t)sl * g.kmagic) >> g.kshift);
          vo = tok * (uint32_t)(g.lda * 2) + colA[j];
        }
        dma(r, sa + (wv * LA + j) * 512, vo);
      }
      if (wv == 0) {
        // the routing weights of the step's rows (64 from its first; past the
        // expert's end: zeros)
        const auto rw = rsrc(g.rowsc + kbeg + k0, (klen - k0) * 4);
        const uint32_t m0 = (uint32_t)reinterpret_cast<uintptr_t>(
            (const __attribute__((address_space(3))) float*)(wst + st * 64));
        const uint32_t vo = (uint32_t)lane * 4;
        asm volatile("buffer_load_dword %0, %1, 0 offen lds" : : "v"(vo), "s"(rw), "{m0}"(m0));
      }
    } else {
      const auto r = rsrc(abase + k0 * g.lda * 2, (klen - k0) * g.lda * 2);
#pragma unroll
      for (int j = 0; j < LA; ++j)
        dma(r, sa + (wv * LA + j) * 512, voA[j]);
    }
    if constexpr (B_KC) {
      const auto r0 = rsrc(bbase0 + k0 * 2, kRange);
      const auto r1 = rsrc(bbase1 + k0 * 2, kRange);
#pragma unroll
      for (int j = 0; j < LB; ++j) {
        const int q = wv * LB + j;
        const uint32_t vo = (tail && k0 + kcB[j] >= kend) ? kOOB : voB[j];
        // gate/up forward: rows BN/2.. of the B tile are the up rows
        const bool up = MODE == GATE_UP_FWD && RPIK * q >= BN / 2;
        dma(up ? r1 : r0, sb + q * 512, vo);
      }
    } else if constexpr (KGROUP) {
      if (GATHER_B && gatherB) {
        // k-row k of the step is expanded row kbeg + k0 + k, i.e. row slot/K of x;
        // k-rows past the expert's end read zeros
        const auto r = rsrc(g.B0, g.gbytes);
        const int32_t* tk = tokr + (kt & 7) * 64;
#pragma unroll
        for (int j = 0; j < LB; ++j) {
          uint32_t vo = kOOB;
          if (k0 + kB[j] < klen) {
            const uint32_t sl = (uint32_t)tk[kB[j]];
            const uint32_t tok = (uint32_t)(((uint64_t)sl * g.kmagic) >> g.kshift);
            vo = tok * (uint32_t)(g.ldb * 2) + colB[j];
          }
          dma(r, sb + (wv * LB + j) * 512, vo);
        }
      } else {
        const auto r = rsrc(bbase0 + k0 * g.ldb * 2, (klen - k0) * g.ldb * 2);
#pragma unroll
        for (int j = 0; j < LB; ++j)
          dma(r, sb + (wv * LB + j) * 512, voB[j]);
      }
    } else {
      // data gradients: B = the expert's weights, K-strided over Kd (= H, or
      // 2F with the gate rows < F and the up rows >= F; F is a multiple of
      // 32, so the k-rows of one instruction lie on one side)
      constexpr int RPI = 64 / (BN / 8);
      const int64_t Fk = MODE == GATE_UP_BWD_DATA ? g.F : g.Kd;
      const auto r0 = rsrc(bbase0 + k0 * g.ldb * 2, (Fk - k0) * g.ldb * 2);
      const auto r1 = rsrc(bbase1 + (k0 - Fk) * g.ldb * 2, (g.Kd - k0) * g.ldb * 2);
#pragma unroll
      for (int j = 0; j < LB; ++j) {
        const int q = wv * LB + j;
        const bool up = MODE == GATE_UP_BWD_DATA && k0 + RPI * q >= Fk;
        dma(up ? r1 : r0, sb + q * 512, voB[j]);
      }
    }
  };

  // LDS read offsets (bf16 elements) of the MFMA fragments, stage 0, sub-step 0
  // K-contiguous operand: one 16-byte read at lds_off(row, 2 kk + lane/32)
  // K-strided operand: two transposing reads at tr_off(i) + (16 kk + 4 r) k-rows
  const int g16 = lane >> 4, i16 = lane & 15;
  auto tr_off = [&](int mbase, int R) {
    const int m = mbase + (g16 & 1) * 16 + 4 * (i16 & 3);
    const int k = (g16 >> 1) * 8 + (i16 >> 2);
    return k * R + (((m >> 3) ^ sw4(k)) << 3) + ((m >> 2) & 1) * 4;
  };
  int trA[TI], trB[TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i) trA[i] = tr_off(wm * (BM / WM) + i * 32, BM);
#pragma unroll
  for (int j = 0; j < TJ; ++j) trB[j] = tr_off(brow(j), BN);
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  auto trread = [](const bf16_t* p) -> v4i16 {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p));
  };
  auto frag_tr = [&](const bf16_t* base, int kk, int R) -> bf16x8 {
    const v4i16 lo = trread(base + (16 * kk) * R);
    const v4i16 hi = trread(base + (16 * kk + 4) * R);
    const v4i16 v[2] = {lo, hi};
    bf16x8 out;
    __builtin_memcpy(&out, v, 16);
    return out;
  };

  // MFMAs of one K step on LDS stage ST; operand fragments of sub-step kk+1 are
  // read while the MFMAs of sub-step kk issue.
  auto compute = [&](auto ST) {
    constexpr int st = decltype(ST)::value;
    const bf16_t* as = smem + st * BM * BK;
    const bf16_t* bs = smem + S * BM * BK + st * BN * BK;
    bf16x8 fa[2][TI], fb[2][TJ];
    auto fetch = [&](int kk, int slot) {
      const int c = kk * 2 + (lane >> 5);
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        if constexpr (!KGROUP) fa[slot][i] = *reinterpret_cast<const bf16x8*>(as + lds_off(arow[i], c));
        else fa[slot][i] = frag_tr(as + trA[i], kk, BM);
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        if constexpr (B_KC) fb[slot][j] = *reinterpret_cast<const bf16x8*>(bs + lds_off(brw[j], c));
        else fb[slot][j] = frag_tr(bs + trB[j], kk, BN);
      }
    };
    // gathered down weight gradient: the A fragments of sub-step kk (k-rows
    // 16 kk + 8 (lane / 32) + 0..7 of the step) times their eight routing weights
    auto scale = [&](int kk, int slot) {
      if constexpr (GATHER_A) {
        if (gatherA) {
          const float4* wp = reinterpret_cast<const float4*>(wst + st * 64 + 16 * kk + 8 * (lane >> 5));
          const float4 w0 = wp[0], w1 = wp[1];
          const float w8[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
          for (int i = 0; i < TI; ++i) fa[slot][i] = scale_bf16x8_each(fa[slot][i], w8);
        }
      }
    };
    fetch(0, 0);
    scale(0, 0);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      if (kk + 1 < BK / 16) fetch(kk + 1, (kk + 1) & 1);
      // keep the reads of sub-step kk+1 ahead of the MFMAs of sub-step kk
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[kk & 1][j], fa[kk & 1][i], acc[i][j], 0, 0, 0);
      // the scaling of sub-step kk+1 issues behind these MFMAs and runs while
      // they execute
      __builtin_amdgcn_sched_barrier(0);
      if (kk + 1 < BK / 16) scale(kk + 1, (kk + 1) & 1);
    }
  };

  // Pipeline: S LDS stages, loads of step t+S-1 issued at step t.  Each step
  // waits for its own loads (the loads of the later steps may stay in
  // flight), then a barrier makes every wave's part of the stage visible and
  // frees the stage of step t-1 for the next loads.
  constexpr int L = LA + LB;
  const int64_t nk = (klen + BK - 1) / BK;
  // K steps run from ks to the end and wrap around.  With krot > 0, the
  // eight tiles that share an A row tile (or a B column tile) start krot
  // steps apart, so one of them fetches each K step's operands from HBM ahead
  // of the others instead of all of them waiting on the same misses.
  const int64_t ks = nk ? ((int64_t)kseed * g.krot) % nk : 0;
  auto rot = [&](int64_t t) -> int64_t { const int64_t u = t + ks; return u < nk ? u : u - nk; };
  // map entries of K step kt (and the next) into ring slot kt % 8, by wave 0,
  // issued at step kt - S - 1 before that step's tile loads: the wait of step
  // kt - S + 1 covers it (it is older than that step's own tile loads), and that
  // step's barrier publishes it before the tile loads of step kt are issued
  auto issue_tok = [&](int64_t kt) {
    if (wv != 0) return;
    const int64_t r0 = kbeg + kt * BK;
    const auto r = rsrc(g.gather + r0, (g.grows - r0) * 4);
    const uint32_t m0 = (uint32_t)reinterpret_cast<uintptr_t>(
        (const __attribute__((address_space(3))) int32_t*)(tokr + (kt & 7) * 64));
    const uint32_t vo = (uint32_t)lane * 4;
    asm volatile("buffer_load_dword %0, %1, 0 offen lds" : : "v"(vo), "s"(r), "{m0}"(m0));
  };
  if ((GATHER_B && gatherB) || (GATHER_A && gatherA)) {
    // the entries of the first S + 1 steps, with plain loads before the pipeline
    static_assert(!GATHER_B || kThreads >= 64, "");
    for (int i = tid; i < (S + 1) * 64; i += kThreads) {
      const int64_t st = i / 64, r0 = kbeg + st * BK + (i % 64);
      tokr[(st & 7) * 64 + (i % 64)] = (st < nk && r0 < g.grows) ? g.gather[r0] : 0;
    }
    __syncthreads();
  }
  auto kstep = [&](auto ST, int64_t kt) {
    constexpr int st = decltype(ST)::value;
    if (kt + S - 2 < nk) __builtin_amdgcn_s_waitcnt(vmcnt_imm(L * (S - 2)));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    // a plain barrier: the LDS reads of step t-1 have completed (their MFMAs
    // consumed them) and the loads of step t were waited for above; the empty
    // statements keep the compiler from moving memory accesses across it
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // (the map entries go before the tile loads: the wait of a later step then
    // covers them without waiting on a tile load issued after them)
    if (((GATHER_B && gatherB) || (GATHER_A && gatherA)) && kt + S + 1 < nk) issue_tok(kt + S + 1);
    if (kt + S - 1 < nk) issue(std::integral_constant<int, (st + S - 1) % S>(), rot(kt + S - 1));
    compute(ST);
  };
#pragma unroll
  for (int t = 0; t < S - 1; ++t)
    if (t < nk) {
      if (t == 0) issue(std::integral_constant<int, 0>(), rot(0));
      if (t == 1) issue(std::integral_constant<int, 1 % S>(), rot(1));
      if (t == 2) issue(std::integral_constant<int, 2 % S>(), rot(2));
    }
  for (int64_t kt = 0; kt < nk; kt += S) {
    kstep(std::integral_constant<int, 0>(), kt);
    if (kt + 1 < nk) kstep(std::integral_constant<int, 1 % S>(), kt + 1);
    if constexpr (S > 2) if (kt + 2 < nk) kstep(std::integral_constant<int, 2 % S>(), kt + 2);
    if constexpr (S > 3) if (kt + 3 < nk) kstep(std::integral_constant<int, 3 % S>(), kt + 3);
  }
  __syncthreads();
  if constexpr (MODE == DOWN_BWD_DATA && !FP8) {
    // gathered: grad_y row r is w_r * grad_out[token]; the row's weight multiplies
    // its fp32 product with W_down (the grad_y path rounds w_r * grad_out to bf16
    // first: one rounding fewer here)
    if (gathered)
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const float wr = g.rowsc[row0 + (arow[i] < rows_valid ? arow[i] : rows_valid - 1)];
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] *= wr;
      }
  }

  }

  // ---- epilogue.
  // The GEMMs accumulate transposed fragments (the MFMA takes the B fragment
  // as its first operand), so acc[i][j][r] holds C(m, n) with
  //   m = wm*(BM/WM) + i*32 + lane%32,  n = brow(j) + (r/4)*8 + (lane/32)*4 + r%4:
  // every lane owns runs of four consecutive columns: the row-grouped GEMMs
  // write them to an LDS staging tile as one 8-byte store, the weight
  // gradients straight to memory as one 16-byte fp32 store.  The K loop
  // ended with a barrier, so the LDS stages are free.
  const int ln = lane & 31, lh = lane >> 5;
  auto tm = [&](int i) { return wm * (BM / WM) + i * 32 + ln; };
  auto tn = [&](int j, int t) { return brow(j) + t * 8 + lh * 4; };
  auto pack4 = [](float a, float b, float c, float d) { return make_uint2(pk_bf16(a, b), pk_bf16(c, d)); };
  constexpr int CP = C::CP, CW = C::CW;
  // cooperative 16-byte row stores of a staged BM x w bf16 tile of pitch p
  // (four LDS reads per thread go out before their stores, so the stores do
  // not each wait out one LDS read)
  auto store_tile_w = [&](const bf16_t* t, int w, int p, bf16_t* dst, int64_t ldd, int64_t ncols, auto NT) {
    constexpr bool nt = decltype(NT)::value;
    typedef unsigned int u32x4s __attribute__((ext_vector_type(4)));
    const int n = BM * (w / 8);
    for (int v0 = 0; v0 < n; v0 += 4 * kThreads) {
      u32x4s val[4];
      int64_t off[4];
      bool ok[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int v = v0 + q * kThreads + tid;
        const int row = v / (w / 8), c8 = (v % (w / 8)) * 8;
        ok[q] = v < n && row < rows_valid && c8 < ncols;
        off[q] = (row0 + row) * ldd + c8;
        if (ok[q]) val[q] = *reinterpret_cast<const u32x4s*>(t + row * p + c8);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (!ok[q]) continue;
        if constexpr (nt) __builtin_nontemporal_store(val[q], reinterpret_cast<u32x4s*>(dst + off[q]));
        else *reinterpret_cast<u32x4s*>(dst + off[q]) = val[q];
      }
    }
  };
  auto store_tile = [&](const bf16_t* t, bf16_t* dst, int64_t ldd, int64_t ncols) {
    store_tile_w(t, CW, CP, dst, ldd, ncols, std::false_type());
  };
  // the same with non-temporal stores, for outputs read back only much later
  // (the saved G and U, read by the backward pass)
  auto store_tile_nt = [&](const bf16_t* t, bf16_t* dst, int64_t ldd, int64_t ncols) {
    store_tile_w(t, CW, CP, dst, ldd, ncols, std::true_type());
  };
  // SwiGLU backward: the saved G and U columns [c0, c0 + W) of the tile's rows
  // into LDS (G at smem, U at smem + BM * P, row pitch P).  A thread's 16-byte
  // loads go out in batches of eight before the batch's first LDS write, so
  // their latencies overlap (a load, wait, write loop pays one memory round
  // trip per chunk); rows past the expert's end repeat its last row, columns
  // past N its last eight.
  auto stage_gu = [&](auto WV, auto PV, int64_t c0) {
    constexpr int W = decltype(WV)::value, P = decltype(PV)::value;
    constexpr int kChunks = 2 * BM * (W / 8), kBatch = 8;
    static_assert(kChunks % (kBatch * kThreads) == 0, "whole batches of eight chunks per thread");
#pragma unroll 1
    for (int b0 = 0; b0 < kChunks; b0 += kBatch * kThreads) {
      uint4 v[kBatch];
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const int idx = b0 + q * kThreads + tid;
        const int t = idx / (BM * (W / 8)), w = idx % (BM * (W / 8));
        const int row = w / (W / 8), c8 = (w % (W / 8)) * 8;
        const int rr = row < rows_valid ? row : rows_valid - 1;
        const int64_t col = c0 + c8 < g.N ? c0 + c8 : g.N - 8;
        v[q] = *reinterpret_cast<const uint4*>(g.aux + (row0 + rr) * 2 * g.F + (t ? g.F : 0) + col);
      }
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const int idx = b0 + q * kThreads + tid;
        const int t = idx / (BM * (W / 8)), w = idx % (BM * (W / 8));
        const int row = w / (W / 8), c8 = (w % (W / 8)) * 8;
        *reinterpret_cast<uint4*>(smem + t * BM * P + row * P + c8) = v[q];
      }
    }
  };
  // MX codes of 32 staged bf16 values (one 32-block of an output row): 32 codes
  // at dst, the scale byte in the step-major word layout (block c32 of the row)
  auto mx_block = [&](const bf16_t* src, int64_t row, int64_t c32, uint8_t* dst) {
    float f[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) unpack8(*reinterpret_cast<const uint4*>(src + 8 * q), f + 8 * q);
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(f[i]));
    const int ex = mx_exponent(m);
    const float inv = mx_inv(ex);
    uint32_t w[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      w[q] = e4m3x4(__fmul_rn(f[4 * q], inv), __fmul_rn(f[4 * q + 1], inv), __fmul_rn(f[4 * q + 2], inv),
                    __fmul_rn(f[4 * q + 3], inv));
    *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint4*>(dst + 16) = make_uint4(w[4], w[5], w[6], w[7]);
    g.smx[((c32 / 4) * g.rowsA + row) * 4 + (c32 & 3)] = (uint8_t)(ex + 127);
  };
  // MX row codes of the staged h (BM rows x BN/2 columns, pitch CP): BN/64
  // 32-blocks per row, one (row, 32-block) per thread at a time (F is a
  // multiple of 128, so the tile's columns are all inside h)
  auto mx_h = [&](const bf16_t* th) {
    constexpr int NB = BN / 64;
    for (int p = tid; p < BM * NB; p += kThreads) {
      const int row = p / NB, b = p % NB;
      if (row < rows_valid)
        mx_block(th + row * CP + 32 * b, row0 + row, (n0 + 32 * b) / 32, g.qmx + (row0 + row) * g.F + n0 + 32 * b);
    }
  };
  if constexpr (MODE == GATE_UP_FWD && C::kEpiGU2) {
    // h and G side by side, then U
    bf16_t* th = smem;
    bf16_t* tg = smem + BM * CP;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ / 2; ++j)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          float gv[4], uv[4], hv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            gv[q] = acc[i][j][4 * t + q];
            uv[q] = acc[i][j + TJ / 2][4 * t + q];
            hv[q] = silu_f(gv[q]) * uv[q];
          }
          const int o = tm(i) * CP + wn * (BN / 2 / WN) + j * 32 + t * 8 + lh * 4;
          *reinterpret_cast<uint2*>(th + o) = pack4(hv[0], hv[1], hv[2], hv[3]);
          *reinterpret_cast<uint2*>(tg + o) = pack4(gv[0], gv[1], gv[2], gv[3]);
        }
    __syncthreads();
    store_tile(th, g.C0 + n0, g.F, g.F - n0);
    store_tile_nt(tg, g.C1 + n0, 2 * g.F, g.F - n0);
    // (the per-token fp8 codes of h, qc, come from the 128 x 128 fp8 tiles only)
    if constexpr (MX)
      if (g.qmx) mx_h(th);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ / 2; ++j)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int o = tm(i) * CP + wn * (BN / 2 / WN) + j * 32 + t * 8 + lh * 4;
          *reinterpret_cast<uint2*>(th + o) = pack4(acc[i][j + TJ / 2][4 * t], acc[i][j + TJ / 2][4 * t + 1],
                                                     acc[i][j + TJ / 2][4 * t + 2], acc[i][j + TJ / 2][4 * t + 3]);
        }
    __syncthreads();
    store_tile_nt(th, g.C1 + g.F + n0, 2 * g.F, g.F - n0);
  } else if constexpr (MODE == GATE_UP_FWD && !C::kEpiOnePass) {
    // h, then G, then U through one staging tile
    bf16_t* ct = smem;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ / 2; ++j)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            float v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float gv = acc[i][j][4 * t + q], uv = acc[i][j + TJ / 2][4 * t + q];
              v[q] = pass == 0 ? silu_f(gv) * uv : (pass == 1 ? gv : uv);
            }
            *reinterpret_cast<uint2*>(ct + tm(i) * CP + wn * (BN / 2 / WN) + j * 32 + t * 8 + lh * 4) =
                pack4(v[0], v[1], v[2], v[3]);
          }
      __syncthreads();
      if (pass == 0) store_tile(ct, g.C0 + n0, g.F, g.F - n0);
      else store_tile_nt(ct, g.C1 + (pass == 2 ? g.F : 0) + n0, 2 * g.F, g.F - n0);
      __syncthreads();
    }
  } else if constexpr (MODE == DOWN_BWD_DATA && !C::kEpiOnePass) {
    // SwiGLU backward one wave column (BN/2 output columns) at a time
    constexpr int WC = BN / WN, CPH = C::CPH;
    bf16_t* tg = smem;
    bf16_t* tu = smem + BM * CPH;
#pragma unroll 1
    for (int pc = 0; pc < WN; ++pc) {
      const int64_t c0 = n0 + pc * WC;
      stage_gu(std::integral_constant<int, WC>(), std::integral_constant<int, CPH>(), c0);
      __syncthreads();
      if (wn == pc) {
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const int o = tm(i) * CPH + tn(j, t) - pc * WC;
              const uint2 gp = *reinterpret_cast<const uint2*>(tg + o);
              const uint2 up = *reinterpret_cast<const uint2*>(tu + o);
              const float gv[4] = {bf2f(gp.x & 0xffffu), bf2f(gp.x >> 16), bf2f(gp.y & 0xffffu), bf2f(gp.y >> 16)};
              const float uv[4] = {bf2f(up.x & 0xffffu), bf2f(up.x >> 16), bf2f(up.y & 0xffffu), bf2f(up.y >> 16)};
              float dg[4], du[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const float c = acc[i][j][4 * t + q];
                const float sg = 1.0f / (1.0f + __expf(-gv[q]));
                dg[q] = c * uv[q] * sg * (1.0f + gv[q] * (1.0f - sg));
                du[q] = c * (gv[q] * sg);
              }
              *reinterpret_cast<uint2*>(tg + o) = pack4(dg[0], dg[1], dg[2], dg[3]);
              *reinterpret_cast<uint2*>(tu + o) = pack4(du[0], du[1], du[2], du[3]);
            }
      }
      __syncthreads();
      store_tile_w(tg, WC, CPH, g.C0 + c0, 2 * g.F, g.N - c0, std::false_type());
      store_tile_w(tu, WC, CPH, g.C0 + g.F + c0, 2 * g.F, g.N - c0, std::false_type());
      __syncthreads();
    }
  } else if constexpr (MODE == GATE_UP_FWD) {
    // h, G and U (BM rows x BN/2 columns each) staged side by side
    bf16_t* th = smem;
    bf16_t* tg = smem + BM * CP;
    bf16_t* tu = smem + 2 * BM * CP;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ / 2; ++j)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          float gv[4], uv[4], hv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            gv[q] = acc[i][j][4 * t + q];
            uv[q] = acc[i][j + TJ / 2][4 * t + q];
            hv[q] = silu_f(gv[q]) * uv[q];
          }
          const int o = tm(i) * CP + wn * (BN / 2 / WN) + j * 32 + t * 8 + lh * 4;
          *reinterpret_cast<uint2*>(th + o) = pack4(hv[0], hv[1], hv[2], hv[3]);
          *reinterpret_cast<uint2*>(tg + o) = pack4(gv[0], gv[1], gv[2], gv[3]);
          *reinterpret_cast<uint2*>(tu + o) = pack4(uv[0], uv[1], uv[2], uv[3]);
        }
    __syncthreads();
    store_tile(th, g.C0 + n0, g.F, g.F - n0);
    store_tile_nt(tg, g.C1 + n0, 2 * g.F, g.F - n0);
    store_tile_nt(tu, g.C1 + g.F + n0, 2 * g.F, g.F - n0);
    if constexpr (FP8) {
      if (g.qmx) mx_h(th);
      if (g.qc) {
        // per-128-token e4m3 codes of the staged bf16 h (the tile's rows are
        // one token slot): thread t takes the column pair 2 (t%32), +1 over
        // rows 16 (t/32) .. +15; the eight row parts meet through LDS
        static_assert(BM == 128 && BN == 128 && kThreads == 256, "one slot, 64 h columns per tile");
        const int pr = tid & 31, rq = tid >> 5;
        uint32_t pv[16];
        float m0 = 0.f, m1 = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = rq * 16 + i;
          pv[i] = r < rows_valid ? *reinterpret_cast<const uint32_t*>(th + r * CP + 2 * pr) : 0u;
          m0 = fmaxf(m0, fabsf(bf2f(pv[i] & 0xffffu)));
          m1 = fmaxf(m1, fabsf(bf2f(pv[i] >> 16)));
        }
        __shared__ float part[8][64];
        part[rq][2 * pr] = m0;
        part[rq][2 * pr + 1] = m1;
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          m0 = fmaxf(m0, part[q][2 * pr]);
          m1 = fmaxf(m1, part[q][2 * pr + 1]);
        }
        const float inv0 = m0 > 0.f ? __fdiv_rn(448.0f, m0) : 0.f;
        const float inv1 = m1 > 0.f ? __fdiv_rn(448.0f, m1) : 0.f;
        uint32_t w0[4], w1[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t* v = pv + 4 * q;
          w0[q] = e4m3x4(__fmul_rn(bf2f(v[0] & 0xffffu), inv0), __fmul_rn(bf2f(v[1] & 0xffffu), inv0),
                         __fmul_rn(bf2f(v[2] & 0xffffu), inv0), __fmul_rn(bf2f(v[3] & 0xffffu), inv0));
          w1[q] = e4m3x4(__fmul_rn(bf2f(v[0] >> 16), inv1), __fmul_rn(bf2f(v[1] >> 16), inv1),
                         __fmul_rn(bf2f(v[2] >> 16), inv1), __fmul_rn(bf2f(v[3] >> 16), inv1));
        }
        const int64_t col = n0 + 2 * pr;
        uint8_t* d0 = g.qc + col * g.ldq + tile_m * 128 + rq * 16;
        *reinterpret_cast<uint4*>(d0) = make_uint4(w0[0], w0[1], w0[2], w0[3]);
        *reinterpret_cast<uint4*>(d0 + g.ldq) = make_uint4(w1[0], w1[1], w1[2], w1[3]);
        if (rq == 0) {
          g.sc[tile_m * g.F + col] = m0 > 0.f ? __fdiv_rn(m0, 448.0f) : 1.0f;
          g.sc[tile_m * g.F + col + 1] = m1 > 0.f ? __fdiv_rn(m1, 448.0f) : 1.0f;
        }
      }
    }
  } else if constexpr (MODE == DOWN_FWD || MODE == GATE_UP_BWD_DATA) {
    bf16_t* ct = smem;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int t = 0; t < 4; ++t)
          *reinterpret_cast<uint2*>(ct + tm(i) * CP + tn(j, t)) =
              pack4(acc[i][j][4 * t], acc[i][j][4 * t + 1], acc[i][j][4 * t + 2], acc[i][j][4 * t + 3]);
    __syncthreads();
    store_tile(ct, g.C0 + n0, g.N, g.N - n0);
  } else if constexpr (MODE == DOWN_BWD_DATA) {
    // SwiGLU backward: the saved G and U of this tile come in as 16-byte rows
    // through LDS; dG and dU replace them in place and leave as 16-byte rows.
    bf16_t* tg = smem;
    bf16_t* tu = smem + BM * CP;
    stage_gu(std::integral_constant<int, BN>(), std::integral_constant<int, CP>(), n0);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int o = tm(i) * CP + tn(j, t);
          const uint2 gp = *reinterpret_cast<const uint2*>(tg + o);
          const uint2 up = *reinterpret_cast<const uint2*>(tu + o);
          const float gv[4] = {bf2f(gp.x & 0xffffu), bf2f(gp.x >> 16), bf2f(gp.y & 0xffffu), bf2f(gp.y >> 16)};
          const float uv[4] = {bf2f(up.x & 0xffffu), bf2f(up.x >> 16), bf2f(up.y & 0xffffu), bf2f(up.y >> 16)};
          float dg[4], du[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float c = acc[i][j][4 * t + q];
            const float sg = 1.0f / (1.0f + __expf(-gv[q]));
            dg[q] = c * uv[q] * sg * (1.0f + gv[q] * (1.0f - sg));
            du[q] = c * (gv[q] * sg);
          }
          *reinterpret_cast<uint2*>(tg + o) = pack4(dg[0], dg[1], dg[2], dg[3]);
          *reinterpret_cast<uint2*>(tu + o) = pack4(du[0], du[1], du[2], du[3]);
        }
    __syncthreads();
    if (g.C0) {
      store_tile(tg, g.C0 + n0, 2 * g.F, g.N - n0);
      store_tile(tu, g.C0 + g.F + n0, 2 * g.F, g.N - n0);
    }
    if constexpr (FP8) {
      if (g.qmx) {
        // MX row codes of dG|dU: four 32-blocks of dG and four of dU per row
        for (int p = tid; p < BM * 8; p += kThreads) {
          const int row = p >> 3, blk = p & 7;
          if (row >= rows_valid) continue;
          const int64_t col = (blk < 4 ? 0 : g.F) + n0 + 32 * (blk & 3);
          mx_block((blk < 4 ? tg : tu) + row * CP + 32 * (blk & 3), row0 + row, col / 32,
                   g.qmx + (row0 + row) * 2 * g.F + col);
        }
      }
      // e4m3 codes of the staged bf16 dG/dU (the values the bf16 output holds),
      // same rule as the quantiser kernels: F is a multiple of 128 and the tile
      // is 128 x 128, so its dG (dU) columns are one whole 128-column block of
      // every row, and its rows one whole 128-token slot (slot = row tile).
      static_assert(BN == 128 && BM == 128 && kThreads == 256, "one block per row, one slot per tile");
      if (g.qr) {
        // rows: 16 lanes per (row, block), 8 columns each
        const int sub = tid & 15;
        for (int p = tid >> 4; p < 2 * BM; p += kThreads / 16) {
          const int row = p >> 1, half = p & 1;
          if (row >= rows_valid) continue;  // the same for the 16 lanes of a group
          float f[8];
          unpack8(*reinterpret_cast<const uint4*>((half ? tu : tg) + row * CP + sub * 8), f);
          float amax = 0.f;
#pragma unroll
          for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(f[q]));
#pragma unroll
          for (int o = 8; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 16));
          const float inv = amax > 0.f ? __fdiv_rn(448.0f, amax) : 0.f;
          const uint32_t lo = e4m3x4(__fmul_rn(f[0], inv), __fmul_rn(f[1], inv), __fmul_rn(f[2], inv),
                                     __fmul_rn(f[3], inv));
          const uint32_t hi = e4m3x4(__fmul_rn(f[4], inv), __fmul_rn(f[5], inv), __fmul_rn(f[6], inv),
                                     __fmul_rn(f[7], inv));
          const int64_t col = (half ? g.F : 0) + n0;
          *reinterpret_cast<uint2*>(g.qr + (row0 + row) * 2 * g.F + col + sub * 8) = make_uint2(lo, hi);
          if (sub == 0) g.sr[(col / 128) * g.rowsA + row0 + row] = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
        }
      }
      if (g.qc) {
        // columns: thread t owns the column pair 2 (t%128), +1 of [dG | dU]
        // over rows 64 (t/128) .. +63 (read once into registers as bf16
        // pairs); the two row halves meet through a small LDS array, rows past
        // the expert's end get code 0
        const int pr = tid & 127, rh = tid >> 7;
        const bf16_t* cs = (pr < BN / 2 ? tg : tu) + 2 * (pr & (BN / 2 - 1)) + rh * 64 * CP;
        uint32_t pv[64];
        float m0 = 0.f, m1 = 0.f;
#pragma unroll
        for (int i = 0; i < 64; ++i) {
          pv[i] = rh * 64 + i < rows_valid ? *reinterpret_cast<const uint32_t*>(cs + i * CP) : 0u;
          m0 = fmaxf(m0, fabsf(bf2f(pv[i] & 0xffffu)));
          m1 = fmaxf(m1, fabsf(bf2f(pv[i] >> 16)));
        }
        __shared__ float part[2 * kThreads];
        part[2 * tid] = m0;
        part[2 * tid + 1] = m1;
        __syncthreads();
        m0 = fmaxf(m0, part[2 * (tid ^ 128)]);
        m1 = fmaxf(m1, part[2 * (tid ^ 128) + 1]);
        const float inv0 = m0 > 0.f ? __fdiv_rn(448.0f, m0) : 0.f;
        const float inv1 = m1 > 0.f ? __fdiv_rn(448.0f, m1) : 0.f;
        const int64_t col = (pr < BN / 2 ? 0 : g.F) + n0 + 2 * (pr & (BN / 2 - 1));
        uint8_t* d0 = g.qc + col * g.ldq + tile_m * 128 + rh * 64;
        uint8_t* d1 = d0 + g.ldq;
#pragma unroll
        for (int r0 = 0; r0 < 64; r0 += 16) {
          uint32_t w0[4], w1[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int i = r0 + 4 * q;
            w0[q] = e4m3x4(__fmul_rn(bf2f(pv[i] & 0xffffu), inv0), __fmul_rn(bf2f(pv[i + 1] & 0xffffu), inv0),
                           __fmul_rn(bf2f(pv[i + 2] & 0xffffu), inv0), __fmul_rn(bf2f(pv[i + 3] & 0xffffu), inv0));
            w1[q] = e4m3x4(__fmul_rn(bf2f(pv[i] >> 16), inv1), __fmul_rn(bf2f(pv[i + 1] >> 16), inv1),
                           __fmul_rn(bf2f(pv[i + 2] >> 16), inv1), __fmul_rn(bf2f(pv[i + 3] >> 16), inv1));
          }
          *reinterpret_cast<uint4*>(d0 + r0) = make_uint4(w0[0], w0[1], w0[2], w0[3]);
          *reinterpret_cast<uint4*>(d1 + r0) = make_uint4(w1[0], w1[1], w1[2], w1[3]);
        }
        if (rh == 0) {
          g.sc[tile_m * 2 * g.F + col] = m0 > 0.f ? __fdiv_rn(m0, 448.0f) : 1.0f;
          g.sc[tile_m * 2 * g.F + col + 1] = m1 > 0.f ? __fdiv_rn(m1, 448.0f) : 1.0f;
        }
      }
    }
  } else if constexpr (kStagedWgrad && WM == 2 && (BM / 2) * (BN + 4) * 4 <= C::kSmem * 2) {
    // weight gradients, fp32, through LDS one wave row (BM/2 output rows) at a
    // time: the waves of that row write their accumulators as 16-byte runs,
    // then every wave stores whole output rows, 64 lanes x 16 bytes per row
    // piece, so each store covers full cache lines (the direct stores below
    // write 32-byte pieces of 32 rows per instruction; measured 4-6% slower)
    constexpr int PW = BN + 4;  // floats per staged row (16 bytes of padding)
    typedef float f32x4nt __attribute__((ext_vector_type(4)));
    float* st = reinterpret_cast<float*>(smem);
#pragma unroll 1
    for (int half = 0; half < 2; ++half) {
      if (wm == half) {
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int t = 0; t < 4; ++t)
              *reinterpret_cast<float4*>(st + (i * 32 + ln) * PW + tn(j, t)) =
                  make_float4(acc[i][j][4 * t], acc[i][j][4 * t + 1], acc[i][j][4 * t + 2], acc[i][j][4 * t + 3]);
      }
      __syncthreads();
      constexpr int kRuns = BN / 4;  // 16-byte runs per row
      for (int v = tid; v < (BM / 2) * kRuns; v += kThreads) {
        const int r = v / kRuns, c4 = (v % kRuns) * 4;
        const int m = half * (BM / 2) + r;
        const int64_t n = n0 + c4;
        if (m >= rows_valid || n >= g.N) continue;
        const float4 val = *reinterpret_cast<const float4*>(st + r * PW + c4);
        float* dst;
        if constexpr (MODE == DOWN_BWD_W) {
          dst = g.W0 + (int64_t)e * g.M * g.N + (row0 + m) * g.N + n;
        } else {
          const int64_t jrow = row0 + m;
          dst = jrow < g.F ? g.W0 + (int64_t)e * g.F * g.N + jrow * g.N + n
                           : g.W1 + (int64_t)e * g.F * g.N + (jrow - g.F) * g.N + n;
        }
        // non-temporal: the gradients are read back only by the optimizer
        // (measured 2-6% faster than plain stores)
        __builtin_nontemporal_store(f32x4nt{val.x, val.y, val.z, val.w}, reinterpret_cast<f32x4nt*>(dst));
      }
      __syncthreads();
    }
  } else {
    // weight gradients, fp32: 16-byte stores of four consecutive columns
    // (N is a multiple of 8, so a run is either wholly inside or outside)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int64_t n = n0 + tn(j, t);
        if (n >= g.N) continue;
#pragma unroll
        for (int i = 0; i < TI; ++i) {
          const int m = tm(i);
          if (m >= rows_valid) continue;
          const float4 v =
              make_float4(acc[i][j][4 * t], acc[i][j][4 * t + 1], acc[i][j][4 * t + 2], acc[i][j][4 * t + 3]);
          if constexpr (MODE == DOWN_BWD_W) {
            *reinterpret_cast<float4*>(g.W0 + (int64_t)e * g.M * g.N + (row0 + m) * g.N + n) = v;
          } else {  // GATE_UP_BWD_W: rows [0, F) -> dWg, [F, 2F) -> dWu
            const int64_t jrow = row0 + m;
            if (jrow < g.F) *reinterpret_cast<float4*>(g.W0 + (int64_t)e * g.F * g.N + jrow * g.N + n) = v;
            else *reinterpret_cast<float4*>(g.W1 + (int64_t)e * g.F * g.N + (jrow - g.F) * g.N + n) = v;
          }
        }
      }
  }
}

template <int MODE, int BM, int BN, bool FP8, int BK = 64, int S = 2, int WM = 2, int WN = 2, bool I8 = false,
          bool MX = false>
moe_status launch_cfg(GemmArgs g, const moe_shape* s, hipStream_t strm) {
  const int64_t ncols = MODE == GATE_UP_FWD ? g.F : g.N;
  const int64_t bn_cols = MODE == GATE_UP_FWD ? BN / 2 : BN;
  g.n_tiles = (ncols + bn_cols - 1) / bn_cols;
  if (MODE == DOWN_BWD_W || MODE == GATE_UP_BWD_W) {
    g.m_tiles = (g.M + BM - 1) / BM;
    // blocks of the per-expert tile grid, one per XCD: kp row blocks x 8/kp
    // column blocks, kp chosen to minimise the operand bytes the eight XCDs
    // read (A strips are read 8/kp times, B strips kp times)
    int best = 1;
    double cost = -1.0;
    for (int kp = 1; kp <= 8; kp *= 2) {
      if (kp > g.m_tiles && kp > 1) break;
      const double c = (double)g.M * (8 / kp) + (double)g.N * kp;
      if (cost < 0 || c < cost) { cost = c; best = kp; }
    }
    g.kp = best;
    g.mch = (g.m_tiles + best - 1) / best;
    g.nch = (g.n_tiles + 8 / best - 1) / (8 / best);
    g.tiles = (int64_t)s->num_experts * g.mch * g.nch * 8;
  } else {
    g.m_tiles = s->capacity / BM + s->num_experts;
    g.tiles = g.m_tiles * g.n_tiles;
    // grouped rasterisation pays once a row tile spans many column tiles
    // (measured: 28 or more column tiles gain 10-30%, 12 or fewer lose a few %)
    g.gm = g.n_tiles >= 16 ? 8 : 1;
    // staggered K starts: measured faster for the forward GEMMs in row-tile
    // order (H = 1536, F = 480: 3-7%), slower for the data gradients and in
    // grouped order, where it stays off
    g.krot = (!FP8 && (MODE == GATE_UP_FWD || MODE == DOWN_FWD) && g.gm == 1) ? 1 : 0;
  }
  if (g.tiles == 0) return MOE_OK;
  const int64_t grid = (g.tiles + 7) / 8 * 8;  // weight gradients: already 8 * E * block
  if (grid > 0x7fffffff) return MOE_ERR_BAD_SHAPE;
  hipLaunchKernelGGL((k_gemm<MODE, BM, BN, FP8, BK, S, WM, WN, I8, MX>), dim3((unsigned)grid),
                     dim3(Cfg<MODE, BM, BN, FP8, BK, S, WM, WN>::kThreads), 0, strm, g);
  return launch_status();
}

template <int MODE, bool FP8 = false, bool I8 = false, bool MX = false>
moe_status launch(GemmArgs& g, const moe_shape* s, hipStream_t strm) {
  // Tile shapes per GEMM kind, chosen by measurement on MI355X (MoE layers at
  // H = 1536 / F = 480 and H = 7168 / F = 2048): 128 x 256 tiles (wave tiles
  // 64 x 128, K step 32, three LDS stages, two workgroups per CU) move a
  // quarter fewer operand bytes per FLOP and win for the gate/up data gradient
  // and both weight gradients, and for the down data gradient once its N (= F)
  // is wide.  A narrow down data gradient has few column tiles; 128 x 128
  // tiles with K step 32 and three stages (48 KB of LDS, three workgroups per
  // CU) give it more tiles and more loads in flight (H = 1536, F = 480: 2-3%
  // faster than two stages; K step 64, or 128 x 256 tiles, 7-9% slower).  The forward GEMMs run 128 x 128 tiles
  // with K step 64 and two stages (two workgroups per CU; three ran the larger
  // MoE layer a third slower) or 256 x 256 tiles (below).  Eight-wave
  // 256 x 256 tiles lost for the backward GEMMs: the SwiGLU backward epilogue
  // runs four wave-column passes, and the weight gradients get too few tiles
  // per expert block.
  if constexpr (MX) {
    // eight-wave 256 x 256 tiles for the forward GEMMs and the gate/up data
    // gradient when they make at least one full round over the CUs (the MX MFMA
    // applies the block scales itself, so the wave tile needs no partial sums)
    if constexpr (MODE == GATE_UP_FWD || MODE == DOWN_FWD || MODE == GATE_UP_BWD_DATA) {
      const int64_t cols256 = MODE == GATE_UP_FWD ? 128 : 256;
      const int64_t ncols = MODE == GATE_UP_FWD ? g.F : g.N;
      const int64_t t256 = (s->capacity / 256 + s->num_experts) * ((ncols + cols256 - 1) / cols256);
      if (t256 >= kCUs) return launch_cfg<MODE, 256, 256, true, 64, 2, 2, 4, false, true>(g, s, strm);
    }
    return launch_cfg<MODE, 128, 128, true, 64, 2, 2, 2, false, true>(g, s, strm);
  } else if constexpr (I8) {
    // as for bf16: a decode-sized batch streams each expert's gate/up weights
    // once on 256 x 256 tiles (integer sums, the scales applied after the loop)
    if constexpr (MODE == GATE_UP_FWD)
      if (s->T * s->K <= 256 * (int64_t)s->num_experts)
        return launch_cfg<MODE, 256, 256, true, 64, 2, 2, 4, true>(g, s, strm);
    return launch_cfg<MODE, 128, 128, true, 64, 2, 2, 2, true>(g, s, strm);
  } else if constexpr (FP8) {
    return launch_cfg<MODE, 128, 128, true>(g, s, strm);
  } else if constexpr (MODE == GATE_UP_BWD_W) {
    // a wide gate/up weight gradient takes eight-wave 256 x 256 tiles (a third
    // fewer operand bytes per FLOP than two 128 x 256 workgroups; measured
    // 5% faster at 2F x H = 4096 x 7168 and 28672 x 4096); an expert grid of
    // few such tiles (page 1: 4 x 6) stays on 128 x 256.  The down weight
    // gradient measured 2% faster on them at H x F = 7168 x 2048 but 5% slower
    // at 4096 x 14336, and stays on 128 x 256.
    const int64_t t256 = ((g.M + 255) / 256) * ((g.N + 255) / 256);
    if (t256 >= 64) return launch_cfg<MODE, 256, 256, false, 32, 3, 2, 4>(g, s, strm);
    return launch_cfg<MODE, 128, 256, false, 32, 3>(g, s, strm);
  } else if constexpr (MODE == GATE_UP_BWD_DATA || MODE == DOWN_BWD_W) {
    return launch_cfg<MODE, 128, 256, false, 32, 3>(g, s, strm);
  } else if constexpr (MODE == DOWN_BWD_DATA) {
    if (g.N >= 1024) return launch_cfg<MODE, 128, 256, false, 32, 3>(g, s, strm);
    return launch_cfg<MODE, 128, 128, false, 32, 3>(g, s, strm);
  } else {
    // forward: 256 x 256 tiles of eight waves (wave tiles 128 x 64, one
    // workgroup of 128 KB LDS per CU) do a fifth more work per memory latency
    // than two 128 x 128 workgroups, but come in quarter as many tiles; they
    // are taken when their rounds of tiles over the CUs, weighted by the 1.7x
    // time one round of them takes, beat the rounds of 128 x 128 tiles
    const int64_t ncols = MODE == GATE_UP_FWD ? g.F : g.N;
    const int64_t cols128 = MODE == GATE_UP_FWD ? 64 : 128, cols256 = 2 * cols128;
    const int64_t t128 = (s->capacity / 128 + s->num_experts) * ((ncols + cols128 - 1) / cols128);
    const int64_t t256 = (s->capacity / 256 + s->num_experts) * ((ncols + cols256 - 1) / cols256);
    const int64_t r128 = (t128 + 2 * kCUs - 1) / (2 * kCUs), r256 = (t256 + kCUs - 1) / kCUs;
    if (17 * r256 < 10 * r128) return launch_cfg<MODE, 256, 256, false, 64, 2, 2, 4>(g, s, strm);
    // a decode-sized batch (at most 256 routed rows per expert on average)
    // streams each expert's gate/up weights once when its rows fit one 256-row
    // tile: 7-8% faster at T = 512, H = 7168, F = 2048, E = 32, K = 8 (the down
    // forward there was 4% slower on them and keeps the 128 x 128 tiles)
    if (MODE == GATE_UP_FWD && s->T * s->K <= 256 * (int64_t)s->num_experts)
      return launch_cfg<MODE, 256, 256, false, 64, 2, 2, 4>(g, s, strm);
    return launch_cfg<MODE, 128, 128, false>(g, s, strm);
  }
}

GemmArgs base_args(const moe_shape* s, const int32_t* prefix) {
  GemmArgs g{};
  g.prefix = prefix;
  g.E = s->num_experts;
  g.F = s->F;
  g.rowsA = s->capacity;
  return g;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_ffn_gate_up_fwd(const moe_shape* s, const void* expand_x,
                                          const void* w_gate, const void* w_up,
                                          const int32_t* ep_recv_counts, void* gate_up_save,
                                          void* h_act, void* stream) {
  moe_status st = check_ffn_shape(s);
  if (st != MOE_OK) return st;
  if (!w_gate || !w_up || !ep_recv_counts) return MOE_ERR_NULL_ARG;
  if (s->capacity == 0) return MOE_OK;
  if (!expand_x || !gate_up_save || !h_act) return MOE_ERR_NULL_ARG;
  GemmArgs g = base_args(s, ep_recv_counts);
  g.A = static_cast<const bf16_t*>(expand_x);
  g.lda = s->H;
  g.B0 = static_cast<const bf16_t*>(w_gate);
  g.B1 = static_cast<const bf16_t*>(w_up);
  g.ldb = s->H;
  g.bstride = s->F * s->H;
  g.N = s->F;
  g.Kd = s->H;
  g.C0 = static_cast<bf16_t*>(h_act);
  g.C1 = static_cast<bf16_t*>(gate_up_save);
  return launch<GATE_UP_FWD>(g, s, as_stream(stream));
}

extern "C" moe_status moe_ffn_gate_up_fwd_gather(const moe_shape* s, const void* x, const int32_t* assist,
                                                 const void* w_gate, const void* w_up,
                                                 const int32_t* ep_recv_counts, void* gate_up_save,
                                                 void* h_act, void* stream) {
  moe_status st = check_ffn_shape(s);
  if (st != MOE_OK) return st;
  if (!w_gate || !w_up || !ep_recv_counts) return MOE_ERR_NULL_ARG;
  // the per-lane byte offsets into x are 31-bit (the top bit marks a load past
  // the end of the contraction)
  if ((s->T + 1) * s->H * 2 > 0x7ffffff0LL) return MOE_ERR_UNSUPPORTED;
  if (s->capacity == 0) return MOE_OK;
  if (!x || !assist || !gate_up_save || !h_act) return MOE_ERR_NULL_ARG;
  GemmArgs g = base_args(s, ep_recv_counts);
  g.A = static_cast<const bf16_t*>(x);
  g.gather = assist + s->T * s->K;  // row -> slot
  g.gK = s->K;
  g.gbytes = s->T * s->H * 2;
  g.lda = s->H;
  g.B0 = static_cast<const bf16_t*>(w_gate);
  g.B1 = static_cast<const bf16_t*>(w_up);
  g.ldb = s->H;
  g.bstride = s->F * s->H;
  g.N = s->F;
  g.Kd = s->H;
  g.C0 = static_cast<bf16_t*>(h_act);
  g.C1 = static_cast<bf16_t*>(gate_up_save);
  return launch<GATE_UP_FWD>(g, s, as_stream(stream));
}

extern "C" moe_status moe_ffn_down_fwd(const moe_shape* s, const void* h_act, const void* w_down,
                                       const int32_t* ep_recv_counts, void* y, void* stream) {
  moe_status st = check_ffn_shape(s);
  if (st != MOE_OK) return st;
  if (!w_down || !ep_recv_counts) return MOE_ERR_NULL_ARG;
  if (s->capacity == 0) return MOE_OK;
  if (!h_act || !y) return MOE_ERR_NULL_ARG;
  GemmArgs g = base_args(s, ep_recv_counts);
  g.A = static_cast<const bf16_t*>(h_act);
  g.lda = s->F;
  g.B0 = static_cast<const bf16_t*>(w_down);
  g.ldb = s->F;
  g.bstride = s->H * s->F;
  g.N = s->H;
  g.Kd = s->F;
  g.C0 = static_cast<bf16_t*>(y);
  return launch<DOWN_FWD>(g, s, as_stream(stream));
}

extern "C" moe_status moe_grouped_ffn(const moe_shape* s, const void* expand_x,
                                      const void* w_gate, const void* w_up, const void* w_down,
                                      const int32_t* ep_recv_counts, void* gate_up_save,
                                      void* h_act, void* y, void* stream) {
  moe_status st = check_ffn_shape(s);
  if (st != MOE_OK) return st;
  if (!w_gate || !w_up || !w_down || !ep_recv_counts) return MOE_ERR_NULL_ARG;
  if (s->capacity > 0 && (!expand_x || !gate_up_save || !h_act || !y)) return MOE_ERR_NULL_ARG;
  st = moe_ffn_gate_up_fwd(s, expand_x, w_gate, w_up, ep_recv_counts, gate_up_save, h_act,
                           stream);
  if (st != MOE_OK) return st;
  return moe_ffn_down_fwd(s, h_act, w_down, ep_recv_counts, y, stream);
}

extern "C" moe_status moe_ffn_down_bwd_data(const moe_shape* s, const void* grad_y,
                                            const void* w_down, const void* gate_up_save,
                                            const int32_t* ep_recv_counts, void* grad_gate_up,
                                            void* stream) {
  moe_status st = check_ffn_shape(s);
  if (st != MOE_OK) return st;
  if (!w_down || !ep_recv_counts) return MOE_ERR_NULL_ARG;
  if (s->capacity == 0) return MOE_OK;
  if (!grad_y || !gate_up_save || !grad_gate_up) return MOE_ERR_NULL_ARG;
  GemmArgs g = base_args(s, ep_recv_counts);
  g.A = static_cast<const bf16_t*>(grad_y);
  g.lda = s->H;
  g.B0 = static_cast<const bf16_t*>(w_down);
  g.ldb = s->F;
  g.bstride = s->H * s->F;
  g.N = s->F;
  g.Kd = s->H;
  g.aux = static_cast<const bf16_t*>(gate_up_save);
  g.C0 = static_cast<bf16_t*>(grad_gate_up);
  return launch<DOWN_BWD_DATA>(g, s, as_stream(stream));
}

extern "C" moe_status moe_ffn_down_bwd_weight(const moe_shape* s, const void* grad_y,
                                              const void* h_act, const int32_t* ep_recv_counts,
                                              float* grad_w_down, void* stream) {
  moe_status st = check_ffn_shape(s);
  if (st != MOE_OK) return st;
  if (!ep_recv_counts || !grad_w_down) return MOE_ERR_NULL_ARG;
  MOE_NEED(grad_y, s->capacity * s->H);
  MOE_NEED(h_act, s->capacity * s->F);
  GemmArgs g = base_args(s, ep_recv_counts);
  g.A = static_cast<const bf16_t*>(grad_y);
  g.lda = s->H;
  g.B0 = static_cast<const bf16_t*>(h_act);
  g.ldb = s->F;
  g.M = s->H;
  g.N = s->F;
  g.W0 = grad_w_down;
  return launch<DOWN_BWD_W>(g, s, as_stream(stream));
}

namespace moe {
namespace {
// slot / K as (slot * kmagic) >> kshift: l = ceil(log2 K), kmagic = floor(2^(32+l) / K) + 1
void set_kdiv(GemmArgs& g, int K) {
  int l = 0;
  while ((1 << l) < K) ++l;
  g.kmagic = (((uint64_t)1 << (32 + l)) / (uint64_t)K) + 1;
  g.kshift = 32 + l;
}
}  // namespace
}  // namespace moe

extern "C" moe_status moe_ffn_down_bwd_data_gather(const moe_shape* s, const void* grad_out, const int32_t* assist,
                                                   const float* row_weights, const void* w_down,
                                                   const void* gate_up_save, const int32_t* ep_recv_counts,
                                                   void* grad_gate_up, void* stream) {
  moe_status st = check_ffn_shape(s);
  if (st != MOE_OK) return st;
  if (!w_down || !ep_recv_counts) return MOE_ERR_NULL_ARG;
  // 31-bit per-lane byte offsets into grad_out (the top bit marks a load past
  // the end of the contraction)
  if ((s->T + 1) * s->H * 2 > 0x7ffffff0LL) return MOE_ERR_UNSUPPORTED;
  if (s->capacity == 0) return MOE_OK;
  if (!grad_out || !assist || !row_weights || !gate_up_save || !grad_gate_up) return MOE_ERR_NULL_ARG;
  GemmArgs g = base_args(s, ep_recv_counts);
  g.A = static_cast<const bf16_t*>(grad_out);
  g.gather = assist + s->T * s->K;  // row -> slot
  g.gK = s->K;
  g.gbytes = s->T * s->H * 2;
  g.rowsc = row_weights;
  g.lda = s->H;
  g.B0 = static_cast<const bf16_t*>(w_down);
  g.ldb = s->F;
  g.bstride = s->H * s->F;
  g.N = s->F;
  g.Kd = s->H;
  g.aux = static_cast<const bf16_t*>(gate_up_save);
  g.C0 = static_cast<bf16_t*>(grad_gate_up);
  return launch<DOWN_BWD_DATA>(g, s, as_stream(stream));
}

extern "C" moe_status moe_ffn_down_bwd_weight_gather(const moe_shape* s, const void* grad_out, const int32_t* assist,
                                                     const float* row_weights, const void* h_act,
                                                     const int32_t* ep_recv_counts, float* grad_w_down,
                                                     void* stream) {
  moe_status st = check_ffn_shape(s);
  if (st != MOE_OK) return st;
  if (!ep_recv_counts || !grad_w_down) return MOE_ERR_NULL_ARG;
  if ((s->T + 1) * s->H * 2 > 0x7ffffff0LL) return MOE_ERR_UNSUPPORTED;
  MOE_NEED(grad_out, s->T * s->H);
  MOE_NEED(assist, s->T * s->K + s->capacity);
  MOE_NEED(row_weights, s->capacity);
  MOE_NEED(h_act, s->capacity * s->F);
  GemmArgs g = base_args(s, ep_recv_counts);
  g.A = static_cast<const bf16_t*>(grad_out);
  g.lda = s->H;
  g.gather = s->capacity > 0 ? assist + s->T * s->K : nullptr;  // row -> slot
  g.gK = s->K;
  g.gbytes = s->T * s->H * 2;
  g.grows = s->capacity;
  g.rowsc = row_weights;
  set_kdiv(g, s->K);
  g.B0 = static_cast<const bf16_t*>(h_act);
  g.ldb = s->F;
  g.M = s->H;
  g.N = s->F;
  g.W0 = grad_w_down;
  return launch<DOWN_BWD_W>(g, s, as_stream(stream));
}

extern "C" moe_status moe_ffn_gate_up_bwd_data(const moe_shape* s, const void* grad_gate_up,
                                               const void* w_gate, const void* w_up,
                                               const int32_t* ep_recv_counts,
                                               void* grad_expand_x, void* stream) {
  moe_status st = check_ffn_shape(s);
  if (st != MOE_OK) return st;
  if (!w_gate || !w_up || !ep_recv_counts) return MOE_ERR_NULL_ARG;
  if (s->capacity == 0) return MOE_OK;
  if (!grad_gate_up || !grad_expand_x) return MOE_ERR_NULL_ARG;
  GemmArgs g = base_args(s, ep_recv_counts);
  g.A = static_cast<const bf16_t*>(grad_gate_up);
  g.lda = 2 * s->F;
  g.B0 = static_cast<const bf16_t*>(w_gate);
  g.B1 = static_cast<const bf16_t*>(w_up);
  g.ldb = s->H;
  g.bstride = s->F * s->H;
  g.N = s->H;
  g.Kd = 2 * s->F;
  g.C0 = static_cast<bf16_t*>(grad_expand_x);
  return launch<GATE_UP_BWD_DATA>(g, s, as_stream(stream));
}

extern "C" moe_status moe_ffn_gate_up_bwd_weight(const moe_shape* s, const void* grad_gate_up,
                                                 const void* expand_x,
                                                 const int32_t* ep_recv_counts,
                                                 float* grad_w_gate, float* grad_w_up,
                                                 void* stream) {
  moe_status st = check_ffn_shape(s);
  if (st != MOE_OK) return st;
  if (!ep_recv_counts || !grad_w_gate || !grad_w_up) return MOE_ERR_NULL_ARG;
  MOE_NEED(grad_gate_up, s->capacity * 2 * s->F);
  MOE_NEED(expand_x, s->capacity * s->H);
  GemmArgs g = base_args(s, ep_recv_counts);
  g.A = static_cast<const bf16_t*>(grad_gate_up);
  g.lda = 2 * s->F;
  g.B0 = static_cast<const bf16_t*>(expand_x);
  g.ldb = s->H;
  g.M = 2 * s->F;
  g.N = s->H;
  g.W0 = grad_w_gate;
  g.W1 = grad_w_up;
  return launch<GATE_UP_BWD_W>(g, s, as_stream(stream));
}

extern "C" moe_status moe_ffn_gate_up_bwd_weight_gather(const moe_shape* s, const void* grad_gate_up,
                                                        const void* x, const int32_t* assist,
                                                        const int32_t* ep_recv_counts, float* grad_w_gate,
                                                        float* grad_w_up, void* stream) {
  moe_status st = check_ffn_shape(s);
  if (st != MOE_OK) return st;
  if (!ep_recv_counts || !grad_w_gate || !grad_w_up) return MOE_ERR_NULL_ARG;
  // the per-lane byte offsets into x are 31-bit (the top bit marks a k-row past
  // the expert's end)
  if ((s->T + 1) * s->H * 2 > 0x7ffffff0LL) return MOE_ERR_UNSUPPORTED;
  MOE_NEED(grad_gate_up, s->capacity * 2 * s->F);
  MOE_NEED(x, s->T * s->H);
  MOE_NEED(assist, s->T * s->K + s->capacity);
  GemmArgs g = base_args(s, ep_recv_counts);
  g.A = static_cast<const bf16_t*>(grad_gate_up);
  g.lda = 2 * s->F;
  g.B0 = static_cast<const bf16_t*>(x);
  g.ldb = s->H;
  g.gather = s->capacity > 0 ? assist + s->T * s->K : nullptr;  // row -> slot
  g.gK = s->K;
  g.gbytes = s->T * s->H * 2;
  g.grows = s->capacity;
  // slot / K = (slot * m) >> (32 + l), l = ceil(log2 K), m = floor(2^(32+l) / K) + 1
  int l = 0;
  while ((1 << l) < s->K) ++l;
  g.kmagic = (((uint64_t)1 << (32 + l)) / (uint64_t)s->K) + 1;
  g.kshift = 32 + l;
  g.M = 2 * s->F;
  g.N = s->H;
  g.W0 = grad_w_gate;
  g.W1 = grad_w_up;
  return launch<GATE_UP_BWD_W>(g, s, as_stream(stream));
}

extern "C" moe_status moe_grouped_ffn_bwd(const moe_shape* s, const void* grad_y,
                                          const void* expand_x, const void* gate_up_save,
                                          const void* h_act, const void* w_gate, const void* w_up,
                                          const void* w_down, const int32_t* ep_recv_counts,
                                          void* grad_gate_up, void* grad_expand_x,
                                          float* grad_w_gate, float* grad_w_up,
                                          float* grad_w_down, void* stream) {
  moe_status st = check_ffn_shape(s);
  if (st != MOE_OK) return st;
  if (!w_gate || !w_up || !w_down || !ep_recv_counts || !grad_w_gate || !grad_w_up ||
      !grad_w_down)
    return MOE_ERR_NULL_ARG;
  if (s->capacity > 0 && (!grad_y || !expand_x || !gate_up_save || !h_act || !grad_gate_up ||
                          !grad_expand_x))
    return MOE_ERR_NULL_ARG;
  st = moe_ffn_down_bwd_data(s, grad_y, w_down, gate_up_save, ep_recv_counts, grad_gate_up,
                             stream);
  if (st != MOE_OK) return st;
  st = moe_ffn_down_bwd_weight(s, grad_y, h_act, ep_recv_counts, grad_w_down, stream);
  if (st != MOE_OK) return st;
  st = moe_ffn_gate_up_bwd_data(s, grad_gate_up, w_gate, w_up, ep_recv_counts, grad_expand_x,
                                stream);
  if (st != MOE_OK) return st;
  return moe_ffn_gate_up_bwd_weight(s, grad_gate_up, expand_x, ep_recv_counts, grad_w_gate,
                                    grad_w_up, stream);
}

// ----------------------------------------------------------------------------- fp8 entries

extern "C" moe_status moe_ffn_gate_up_fwd_fp8(const moe_shape* s, const uint8_t* xq,
                                              const float* xs, const uint8_t* wgq,
                                              const float* wgs, const uint8_t* wuq,
                                              const float* wus, const int32_t* ep_recv_counts,
                                              void* gate_up_save, void* h_act, void* stream) {
  moe_status st = check_fp8_shape(s);
  if (st != MOE_OK) return st;
  if (!wgq || !wgs || !wuq || !wus || !ep_recv_counts) return MOE_ERR_NULL_ARG;
  if (s->capacity == 0) return MOE_OK;
  if (!xq || !xs || !gate_up_save || !h_act) return MOE_ERR_NULL_ARG;
  GemmArgs g = base_args(s, ep_recv_counts);
  g.qA = xq;
  g.sA = xs;
  g.lda = s->H;
  g.qB0 = wgq;
  g.qB1 = wuq;
  g.sB0 = wgs;
  g.sB1 = wus;
  g.ldb = s->H;
  g.bstride = s->F * s->H;
  g.sbe = (s->F / 128) * (s->H / 128);  // (E, F/128, H/128): [e][n-block][k-block]
  g.sbn = s->H / 128;
  g.sbk = 1;
  g.N = s->F;
  g.Kd = s->H;
  g.C0 = static_cast<bf16_t*>(h_act);
  g.C1 = static_cast<bf16_t*>(gate_up_save);
  return launch<GATE_UP_FWD, true>(g, s, as_stream(stream));
}

extern "C" moe_status moe_ffn_gate_up_fwd_fp8_quant(const moe_shape* s, const uint8_t* xq,
                                                    const float* xs, const uint8_t* wgq,
                                                    const float* wgs, const uint8_t* wuq,
                                                    const float* wus, const int32_t* ep_recv_counts,
                                                    void* gate_up_save, void* h_act, uint8_t* hq_t,
                                                    float* hs_t, void* stream) {
  moe_status st = check_fp8_shape(s);
  if (st != MOE_OK) return st;
  if (!wgq || !wgs || !wuq || !wus || !ep_recv_counts) return MOE_ERR_NULL_ARG;
  if (s->capacity == 0) return MOE_OK;
  if (!xq || !xs || !gate_up_save || !h_act || !hq_t || !hs_t) return MOE_ERR_NULL_ARG;
  GemmArgs g = base_args(s, ep_recv_counts);
  g.qA = xq;
  g.sA = xs;
  g.lda = s->H;
  g.qB0 = wgq;
  g.qB1 = wuq;
  g.sB0 = wgs;
  g.sB1 = wus;
  g.ldb = s->H;
  g.bstride = s->F * s->H;
  g.sbe = (s->F / 128) * (s->H / 128);
  g.sbn = s->H / 128;
  g.sbk = 1;
  g.N = s->F;
  g.Kd = s->H;
  g.C0 = static_cast<bf16_t*>(h_act);
  g.C1 = static_cast<bf16_t*>(gate_up_save);
  g.qc = hq_t;
  g.sc = hs_t;
  g.ldq = 128 * (s->capacity / 128 + s->num_experts);
  return launch<GATE_UP_FWD, true>(g, s, as_stream(stream));
}

extern "C" moe_status moe_ffn_down_fwd_fp8(const moe_shape* s, const uint8_t* hq, const float* hs,
                                           const uint8_t* wdq, const float* wds,
                                           const int32_t* ep_recv_counts, void* y, void* stream) {
  moe_status st = check_fp8_shape(s);
  if (st != MOE_OK) return st;
  if (!wdq || !wds || !ep_recv_counts) return MOE_ERR_NULL_ARG;
  if (s->capacity == 0) return MOE_OK;
  if (!hq || !hs || !y) return MOE_ERR_NULL_ARG;
  GemmArgs g = base_args(s, ep_recv_counts);
  g.qA = hq;
  g.sA = hs;
  g.lda = s->F;
  g.qB0 = wdq;
  g.sB0 = wds;
  g.ldb = s->F;
  g.bstride = s->H * s->F;
  g.sbe = (s->H / 128) * (s->F / 128);  // (E, H/128, F/128): [e][n-block][k-block]
  g.sbn = s->F / 128;
  g.sbk = 1;
  g.N = s->H;
  g.Kd = s->F;
  g.C0 = static_cast<bf16_t*>(y);
  return launch<DOWN_FWD, true>(g, s, as_stream(stream));
}

extern "C" moe_status moe_ffn_down_bwd_data_fp8(const moe_shape* s, const uint8_t* dyq,
                                                const float* dys, const uint8_t* wdq_t,
                                                const float* wds, const void* gate_up_save,
                                                const int32_t* ep_recv_counts, void* grad_gate_up,
                                                void* stream) {
  moe_status st = check_fp8_shape(s);
  if (st != MOE_OK) return st;
  if (!wdq_t || !wds || !ep_recv_counts) return MOE_ERR_NULL_ARG;
  if (s->capacity == 0) return MOE_OK;
  if (!dyq || !dys || !gate_up_save || !grad_gate_up) return MOE_ERR_NULL_ARG;
  GemmArgs g = base_args(s, ep_recv_counts);
  g.qA = dyq;
  g.sA = dys;
  g.lda = s->H;
  g.qB0 = wdq_t;  // (E, F, H): row f of expert e holds Wd_e[:, f]
  g.sB0 = wds;    // scales of Wd (E, H/128, F/128): [e][k-block (h)][n-block (f)]
  g.ldb = s->H;
  g.bstride = s->F * s->H;
  g.sbe = (s->H / 128) * (s->F / 128);
  g.sbn = 1;
  g.sbk = s->F / 128;
  g.N = s->F;
  g.Kd = s->H;
  g.aux = static_cast<const bf16_t*>(gate_up_save);
  g.C0 = static_cast<bf16_t*>(grad_gate_up);
  return launch<DOWN_BWD_DATA, true>(g, s, as_stream(stream));
}

extern "C" moe_status moe_ffn_down_bwd_data_fp8_quant(const moe_shape* s, const uint8_t* dyq,
                                                      const float* dys, const uint8_t* wdq_t,
                                                      const float* wds, const void* gate_up_save,
                                                      const int32_t* ep_recv_counts, void* grad_gate_up,
                                                      uint8_t* dguq, float* dgus, uint8_t* dguq_t,
                                                      float* dgus_t, void* stream) {
  moe_status st = check_fp8_shape(s);
  if (st != MOE_OK) return st;
  if (!wdq_t || !wds || !ep_recv_counts) return MOE_ERR_NULL_ARG;
  if (!grad_gate_up && !dguq && !dguq_t) return MOE_ERR_NULL_ARG;  // nothing to produce
  if (!dguq != !dgus || !dguq_t != !dgus_t) return MOE_ERR_NULL_ARG;
  if (s->capacity == 0) return MOE_OK;
  if (!dyq || !dys || !gate_up_save) return MOE_ERR_NULL_ARG;
  GemmArgs g = base_args(s, ep_recv_counts);
  g.qA = dyq;
  g.sA = dys;
  g.lda = s->H;
  g.qB0 = wdq_t;
  g.sB0 = wds;
  g.ldb = s->H;
  g.bstride = s->F * s->H;
  g.sbe = (s->H / 128) * (s->F / 128);
  g.sbn = 1;
  g.sbk = s->F / 128;
  g.N = s->F;
  g.Kd = s->H;
  g.aux = static_cast<const bf16_t*>(gate_up_save);
  g.C0 = static_cast<bf16_t*>(grad_gate_up);
  g.qr = dguq;
  g.sr = dgus;
  g.qc = dguq_t;
  g.sc = dgus_t;
  g.ldq = 128 * (s->capacity / 128 + s->num_experts);
  return launch<DOWN_BWD_DATA, true>(g, s, as_stream(stream));
}

extern "C" moe_status moe_ffn_gate_up_bwd_data_fp8(const moe_shape* s, const uint8_t* dguq,
                                                   const float* dgus, const uint8_t* wgq_t,
                                                   const float* wgs, const uint8_t* wuq_t,
                                                   const float* wus, const int32_t* ep_recv_counts,
                                                   void* grad_expand_x, void* stream) {
  moe_status st = check_fp8_shape(s);
  if (st != MOE_OK) return st;
  if (!wgq_t || !wgs || !wuq_t || !wus || !ep_recv_counts) return MOE_ERR_NULL_ARG;
  if (s->capacity == 0) return MOE_OK;
  if (!dguq || !dgus || !grad_expand_x) return MOE_ERR_NULL_ARG;
  GemmArgs g = base_args(s, ep_recv_counts);
  g.qA = dguq;
  g.sA = dgus;
  g.lda = 2 * s->F;
  g.qB0 = wgq_t;  // (E, H, F): row h of expert e holds Wg_e[:, h]
  g.qB1 = wuq_t;
  g.sB0 = wgs;    // scales of Wg (E, F/128, H/128): [e][k-block (f)][n-block (h)]
  g.sB1 = wus;
  g.ldb = s->F;
  g.bstride = s->F * s->H;
  g.sbe = (s->F / 128) * (s->H / 128);
  g.sbn = 1;
  g.sbk = s->H / 128;
  g.N = s->H;
  g.Kd = 2 * s->F;
  g.C0 = static_cast<bf16_t*>(grad_expand_x);
  return launch<GATE_UP_BWD_DATA, true>(g, s, as_stream(stream));
}

// fp8 weight gradients on per-128-token codes (moe_quant_cols_fp8 layout): row
// r of a code matrix holds column r of the activation, the expert's token
// slots along it, ld = 128 * (capacity/128 + E) codes; scales (slots, D).
namespace {
moe_status check_wgrad_fp8(const moe_shape* s, int64_t ncols) {
  moe_status st = check_fp8_shape(s);
  if (st != MOE_OK) return st;
  const int64_t ldq = 128 * (s->capacity / 128 + s->num_experts);
  // code rows are addressed with 32-bit byte offsets from the K step's base
  if (ncols * ldq + 128 >= (int64_t)0x7ffffff0) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}
}  // namespace

extern "C" moe_status moe_ffn_down_bwd_weight_fp8(const moe_shape* s, const uint8_t* dyq_t,
                                                  const float* dys, const uint8_t* hq_t,
                                                  const float* hs, const int32_t* ep_recv_counts,
                                                  float* grad_w_down, void* stream) {
  moe_status st = check_wgrad_fp8(s, s ? (s->H > s->F ? s->H : s->F) : 0);
  if (st != MOE_OK) return st;
  if (!ep_recv_counts || !grad_w_down) return MOE_ERR_NULL_ARG;
  if (s->capacity > 0 && (!dyq_t || !dys || !hq_t || !hs)) return MOE_ERR_NULL_ARG;
  GemmArgs g = base_args(s, ep_recv_counts);
  const int64_t ldq = 128 * (s->capacity / 128 + s->num_experts);
  g.qA = dyq_t;
  g.sA = dys;
  g.lda = ldq;
  g.qB0 = hq_t;
  g.sB0 = hs;
  g.ldb = ldq;
  g.M = s->H;
  g.N = s->F;
  g.W0 = grad_w_down;
  return launch<DOWN_BWD_W, true>(g, s, as_stream(stream));
}

extern "C" moe_status moe_ffn_gate_up_bwd_weight_fp8(const moe_shape* s, const uint8_t* dguq_t,
                                                     const float* dgus, const uint8_t* xq_t,
                                                     const float* xs, const int32_t* ep_recv_counts,
                                                     float* grad_w_gate, float* grad_w_up,
                                                     void* stream) {
  moe_status st = check_wgrad_fp8(s, s ? (2 * s->F > s->H ? 2 * s->F : s->H) : 0);
  if (st != MOE_OK) return st;
  if (!ep_recv_counts || !grad_w_gate || !grad_w_up) return MOE_ERR_NULL_ARG;
  if (s->capacity > 0 && (!dguq_t || !dgus || !xq_t || !xs)) return MOE_ERR_NULL_ARG;
  GemmArgs g = base_args(s, ep_recv_counts);
  const int64_t ldq = 128 * (s->capacity / 128 + s->num_experts);
  g.qA = dguq_t;
  g.sA = dgus;
  g.lda = ldq;
  g.qB0 = xq_t;
  g.sB0 = xs;
  g.ldb = ldq;
  g.M = 2 * s->F;
  g.N = s->H;
  g.W0 = grad_w_gate;
  g.W1 = grad_w_up;
  return launch<GATE_UP_BWD_W, true>(g, s, as_stream(stream));
}

// ----------------------------------------------------------------------------- int8 entries

extern "C" moe_status moe_ffn_gate_up_fwd_int8(const moe_shape* s, const int8_t* xq, const float* xs,
                                               const int8_t* wgq, const float* wgs, const int8_t* wuq,
                                               const float* wus, const int32_t* ep_recv_counts,
                                               void* gate_up_save, void* h_act, void* stream) {
  moe_status st = check_fp8_shape(s);
  if (st != MOE_OK) return st;
  if (!wgq || !wgs || !wuq || !wus || !ep_recv_counts) return MOE_ERR_NULL_ARG;
  if (s->capacity == 0) return MOE_OK;
  if (!xq || !xs || !gate_up_save || !h_act) return MOE_ERR_NULL_ARG;
  GemmArgs g = base_args(s, ep_recv_counts);
  g.qA = reinterpret_cast<const uint8_t*>(xq);
  g.sA = xs;  // one scale per row
  g.lda = s->H;
  g.qB0 = reinterpret_cast<const uint8_t*>(wgq);
  g.qB1 = reinterpret_cast<const uint8_t*>(wuq);
  g.sB0 = wgs;  // (E, F): one scale per output channel
  g.sB1 = wus;
  g.ldb = s->H;
  g.bstride = s->F * s->H;
  g.N = s->F;
  g.Kd = s->H;
  g.C0 = static_cast<bf16_t*>(h_act);
  g.C1 = static_cast<bf16_t*>(gate_up_save);
  return launch<GATE_UP_FWD, true, true>(g, s, as_stream(stream));
}

extern "C" moe_status moe_ffn_down_fwd_int8(const moe_shape* s, const int8_t* hq, const float* hs,
                                            const int8_t* wdq, const float* wds,
                                            const int32_t* ep_recv_counts, void* y, void* stream) {
  moe_status st = check_fp8_shape(s);
  if (st != MOE_OK) return st;
  if (!wdq || !wds || !ep_recv_counts) return MOE_ERR_NULL_ARG;
  if (s->capacity == 0) return MOE_OK;
  if (!hq || !hs || !y) return MOE_ERR_NULL_ARG;
  GemmArgs g = base_args(s, ep_recv_counts);
  g.qA = reinterpret_cast<const uint8_t*>(hq);
  g.sA = hs;
  g.lda = s->F;
  g.qB0 = reinterpret_cast<const uint8_t*>(wdq);
  g.sB0 = wds;  // (E, H)
  g.ldb = s->F;
  g.bstride = s->H * s->F;
  g.N = s->H;
  g.Kd = s->F;
  g.C0 = static_cast<bf16_t*>(y);
  return launch<DOWN_FWD, true, true>(g, s, as_stream(stream));
}

// ----------------------------------------------------------------------------- MX (microscaled fp8) entries

extern "C" moe_status moe_ffn_gate_up_fwd_mx(const moe_shape* s, const uint8_t* xq, const uint8_t* xs,
                                             const uint8_t* wgq, const uint8_t* wgs, const uint8_t* wuq,
                                             const uint8_t* wus, const int32_t* ep_recv_counts,
                                             void* gate_up_save, void* h_act, uint8_t* hq, uint8_t* hs,
                                             void* stream) {
  moe_status st = check_fp8_shape(s);
  if (st != MOE_OK) return st;
  if (!wgq || !wgs || !wuq || !wus || !ep_recv_counts) return MOE_ERR_NULL_ARG;
  if (!hq != !hs) return MOE_ERR_NULL_ARG;
  if (s->capacity == 0) return MOE_OK;
  if (!xq || !xs || !gate_up_save || !h_act) return MOE_ERR_NULL_ARG;
  GemmArgs g = base_args(s, ep_recv_counts);
  g.qA = xq;
  g.lda = s->H;
  g.qB0 = wgq;
  g.qB1 = wuq;
  g.ldb = s->H;
  g.bstride = s->F * s->H;
  g.mA = xs;
  g.mrA = s->capacity;
  g.mB0 = wgs;  // words (H/128, E*F)
  g.mB1 = wus;
  g.mrB = (int64_t)s->num_experts * s->F;
  g.mbe = s->F;
  g.N = s->F;
  g.Kd = s->H;
  g.C0 = static_cast<bf16_t*>(h_act);
  g.C1 = static_cast<bf16_t*>(gate_up_save);
  g.qmx = hq;
  g.smx = hs;
  return launch<GATE_UP_FWD, true, false, true>(g, s, as_stream(stream));
}

extern "C" moe_status moe_ffn_down_fwd_mx(const moe_shape* s, const uint8_t* hq, const uint8_t* hs,
                                          const uint8_t* wdq, const uint8_t* wds, const int32_t* ep_recv_counts,
                                          void* y, void* stream) {
  moe_status st = check_fp8_shape(s);
  if (st != MOE_OK) return st;
  if (!wdq || !wds || !ep_recv_counts) return MOE_ERR_NULL_ARG;
  if (s->capacity == 0) return MOE_OK;
  if (!hq || !hs || !y) return MOE_ERR_NULL_ARG;
  GemmArgs g = base_args(s, ep_recv_counts);
  g.qA = hq;
  g.lda = s->F;
  g.qB0 = wdq;
  g.ldb = s->F;
  g.bstride = s->H * s->F;
  g.mA = hs;
  g.mrA = s->capacity;
  g.mB0 = wds;  // words (F/128, E*H)
  g.mrB = (int64_t)s->num_experts * s->H;
  g.mbe = s->H;
  g.N = s->H;
  g.Kd = s->F;
  g.C0 = static_cast<bf16_t*>(y);
  return launch<DOWN_FWD, true, false, true>(g, s, as_stream(stream));
}

extern "C" moe_status moe_ffn_down_bwd_data_mx(const moe_shape* s, const uint8_t* dyq, const uint8_t* dys,
                                               const uint8_t* wdq_t, const uint8_t* wds_t,
                                               const void* gate_up_save, const int32_t* ep_recv_counts,
                                               void* grad_gate_up, uint8_t* dguq, uint8_t* dgus,
                                               void* stream) {
  moe_status st = check_fp8_shape(s);
  if (st != MOE_OK) return st;
  if (!wdq_t || !wds_t || !ep_recv_counts) return MOE_ERR_NULL_ARG;
  if (!dguq != !dgus || (!grad_gate_up && !dguq)) return MOE_ERR_NULL_ARG;
  if (s->capacity == 0) return MOE_OK;
  if (!dyq || !dys || !gate_up_save) return MOE_ERR_NULL_ARG;
  GemmArgs g = base_args(s, ep_recv_counts);
  g.qA = dyq;
  g.lda = s->H;
  g.qB0 = wdq_t;  // (E, F, H): row f holds Wd_e[:, f]
  g.ldb = s->H;
  g.bstride = s->F * s->H;
  g.mA = dys;
  g.mrA = s->capacity;
  g.mB0 = wds_t;  // words (H/128, E*F)
  g.mrB = (int64_t)s->num_experts * s->F;
  g.mbe = s->F;
  g.N = s->F;
  g.Kd = s->H;
  g.aux = static_cast<const bf16_t*>(gate_up_save);
  g.C0 = static_cast<bf16_t*>(grad_gate_up);
  g.qmx = dguq;
  g.smx = dgus;
  return launch<DOWN_BWD_DATA, true, false, true>(g, s, as_stream(stream));
}

extern "C" moe_status moe_ffn_gate_up_bwd_data_mx(const moe_shape* s, const uint8_t* dguq, const uint8_t* dgus,
                                                  const uint8_t* wgq_t, const uint8_t* wgs_t, const uint8_t* wuq_t,
                                                  const uint8_t* wus_t, const int32_t* ep_recv_counts,
                                                  void* grad_expand_x, void* stream) {
  moe_status st = check_fp8_shape(s);
  if (st != MOE_OK) return st;
  if (!wgq_t || !wgs_t || !wuq_t || !wus_t || !ep_recv_counts) return MOE_ERR_NULL_ARG;
  if (s->capacity == 0) return MOE_OK;
  if (!dguq || !dgus || !grad_expand_x) return MOE_ERR_NULL_ARG;
  GemmArgs g = base_args(s, ep_recv_counts);
  g.qA = dguq;
  g.lda = 2 * s->F;
  g.qB0 = wgq_t;  // (E, H, F): row h holds Wg_e[:, h]
  g.qB1 = wuq_t;
  g.ldb = s->F;
  g.bstride = s->F * s->H;
  g.mA = dgus;
  g.mrA = s->capacity;
  g.mB0 = wgs_t;  // words (F/128, E*H)
  g.mB1 = wus_t;
  g.mrB = (int64_t)s->num_experts * s->H;
  g.mbe = s->H;
  g.N = s->H;
  g.Kd = 2 * s->F;
  g.C0 = static_cast<bf16_t*>(grad_expand_x);
  return launch<GATE_UP_BWD_DATA, true, false, true>(g, s, as_stream(stream));
}
