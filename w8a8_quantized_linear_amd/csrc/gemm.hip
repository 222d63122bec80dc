// Integer (and E4M3FN) GEMM with fused epilogues for gfx950 (stages 2 and 3 of
// the W8A8 path).
//
// What it computes: acc[m][n] = sum_k a[m][k] * b[n][k] over int8 codes (exact
// int32) or E4M3FN codes (fp32 accumulation), followed by
//   kRawI32 : acc as int32;
//   kDequant: bf16(acc * s_tok[m] * s_ch[n] + bias[n])  -- the scale and bias
//             fusion of the INT8 GEMM epilogue ("CLEF Calibrated INT8 ConvRot"
//             card, Benefits list);
//   kSwiglu : bf16(silu(g) * u) with g, u the dequantized values of packed rows
//             n and N + n -- the paired gate/up epilogue ("Loading CLEF INT8",
//             fuse_mlp; gate/up packed into one weight at load time).
// The bf16 outputs go through LDS so that stores cover whole row segments.
//
// Design.  Both operands are K-contiguous ("NT"), so MFMA operands load with no
// transpose.  A workgroup of WGM x WGN waves owns a BM (tokens) x BN (weight
// rows) tile; each wave accumulates a (BM/WGM) x (BN/WGN) sub-tile from 32x32
// MFMA blocks: v_mfma_i32_32x32x32_i8 for int8; E4M3FN operands are widened
// exactly to bf16 in registers and go through v_mfma_f32_32x32x16_bf16, because
// the gfx950 fp8 MFMAs sum their products less accurately than fp32 accumulation
// (measured on the device by tests/test_gpu_fp8_mfma_accuracy.py: errors up to
// ~3e-4 of the output rms at K = 4096 for the 32x32x16 and scaled 32x32x64 fp8
// instructions, chained or with fp32 partial sums, which fails the bf16 output
// tolerance on outputs near zero), while the bf16 MFMA on the same values is
// accurate to fp32 rounding.  The weight fragment is the MFMA's A operand and the token fragment
// its B operand, so a lane ends up holding four consecutive output columns of
// one token row.
//
// Per-wave LDS traffic is (rows_m + rows_n) x K bytes for 2 rows_m rows_n K
// ops, so large wave tiles need less LDS bandwidth per MFMA.  K advances BK = 64
// bytes per stage through a ring of NST LDS buffers filled by direct-to-LDS
// loads (global_load_lds_dwordx4: no staging registers, no LDS write
// instructions), issued NST - 2 stages ahead of use; one barrier per stage.
// LDS rows are XOR-swizzled in 16-byte units so the MFMA operand reads are
// bank-conflict free.  Operands may be row-major or in the packed layout of
// 32-row x 64-byte blocks, in which every 32 rows of a stage are one contiguous
// 2 KiB read instead of 32 separate 64-byte pieces.
//
// Tile order: the hardware deals workgroups round-robin to the 8 XCDs (each
// with its own L2), so block ids are remapped to give every XCD a contiguous
// range of tiles, walked in groups of kGroupM token tiles so that concurrently
// running tiles on one XCD share their token and weight panels in its L2.
//
// The 256 x 256 tile (one workgroup per CU) runs persistent (gemm_persist):
// each workgroup walks several tiles and its operand ring runs on from one tile
// into the next, so the next tile's first stages load while this tile's
// epilogue runs; the smaller tiles (two workgroups per CU) launch one
// workgroup per tile (gemm_tile), where one workgroup's epilogue overlaps the
// other's K loop.
#include <algorithm>
#include <type_traits>

#include "epilogue_math.h"
#include "internal.h"

namespace w8a8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));  // staging (HIP's uint4 is a union
                                                              // struct that defeats SROA)
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kXcds = 8;
constexpr int kCus = 256;
constexpr int kGroupM = 4;

// 16-byte chunk c of LDS row r (CH chunks per row) is stored at chunk position
// c ^ swz_key<CH>(r).  An MFMA operand read (ds_read_b128) has lanes 0-31 fetch
// chunk c of 32 consecutive rows and lanes 32-63 chunk c + 1 of the same rows.
// With 64-byte rows the key (r ^ (r >> 2)) & 3 makes these reads conflict-free
// on this chip's LDS: 4 cycles per read and no bank-conflict cycles, measured
// with the LDS pattern probe and in the GEMM itself, where the earlier key
// ((r >> 1) ^ (r >> 3)) & 3 took 8 cycles (2-way conflicts).
template <int CH>
__device__ __forceinline__ int swz_key(int r) {
  static_assert(CH == 4, "64-byte LDS rows");
  return (r ^ (r >> 2)) & 3;
}
template <int CH>
__device__ __forceinline__ int swz(int r, int c) { return (r * CH + (c ^ swz_key<CH>(r))) * 16; }

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Eight E4M3FN codes -> eight bf16 values (exact: every E4M3FN value, subnormals
// included, is a bf16 value).
__device__ __forceinline__ v8bf e4m3x8_to_bf16(u32x2 v) {
  const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v.x, 1.0f, false);
  const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v.x, 1.0f, true);
  const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v.y, 1.0f, false);
  const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v.y, 1.0f, true);
  const v4bf lo = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
  const v4bf hi = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Tile index within the launch -> (tile_m, tile_n), walked in groups of kGroupM
// token tiles.
__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int per_group = kGroupM * tiles_n;
  const int group = t / per_group, first_m = group * kGroupM;
  const int gsize = min(kGroupM, tiles_m - first_m);
  const int in = t % per_group;
  tm = first_m + in % gsize;
  tn = in / gsize;
}

// Block id -> (tile_m, tile_n): contiguous tile ranges per XCD, grouped along M.
__device__ __forceinline__ void tile_of_block(int bid, int nblocks, int tiles_m, int tiles_n,
                                              int& tm, int& tn) {
  const int q = nblocks / kXcds, r = nblocks % kXcds;
  const int xcd = bid % kXcds, idx = bid / kXcds;
  const int t = (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
  tile_coords(t, tiles_m, tiles_n, tm, tn);
}

// 16 bytes from global memory straight into LDS.  The LDS address must be
// wave-uniform (it goes to M0); lane i's bytes land at lds + 16 * i.  (The
// builtin exists only for the device; the host pass just needs the kernel stub.)
__device__ __forceinline__ void lds_dma16(const uint8_t* g, uint8_t* l) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
#endif
}

// Wait until at most n of this thread's vector-memory loads are outstanding.
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// Raw int32 epilogue of one wave's (TM x TN) 32x32 blocks, stored from
// registers (the int32 output exists for the exactness tests only).  32x32
// block layout: lane l holds token column l % 32 and, in registers 4q .. 4q+3,
// weight rows 8q + 4 * (l / 32) + 0..3 of the block.
// Workgroup barrier for LDS reuse: this wave's LDS accesses are complete
// (lgkmcnt(0)) before it arrives, but its global loads and stores may still be
// in flight (__syncthreads would wait for those too).  The empty asm keeps the
// compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int TM, int TN, int WTM, int WTN, typename Acc>
__device__ __forceinline__ void store_tile_i32(const Acc (&acc)[TN][TM], int32_t* __restrict__ out, int64_t M,
                                               int64_t N, int64_t mb, int64_t nb, int wm, int wn, int frag_row,
                                               int frag_half) {
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int64_t m = mb + wm * WTM + tm * 32 + frag_row;
    if (m >= M) continue;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t n0 = nb + wn * WTN + tn * 32 + 8 * q + 4 * frag_half;
        if (n0 >= N) continue;
        const v16i& v = reinterpret_cast<const v16i&>(acc[tn][tm]);
        *reinterpret_cast<int4*>(out + m * N + n0) = make_int4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
      }
  }
}

// bf16 epilogues (kDequant, kSwiglu) staged through LDS.  In the MFMA layout a
// lane holds 4 consecutive columns of one row, so a direct store instruction
// writes 16 bytes into each of 32 rows -- 32 partial cache lines per
// instruction, which held the output to ~1 TB/s (a 1,502 x 4,096 GEMM at K = 128
// took 13 us).  Instead each wave writes its (WTM x COLS) bf16 sub-tile into its
// own LDS region (rows of COLS * 2 bytes, 16-byte chunks XOR-swizzled by row so
// the 32 rows of a write spread over the banks), then reads it back 16 bytes
// per lane with consecutive lanes along a row, so each store instruction
// covers 64 / (COLS / 8) whole row segments.  The region is part of the operand
// ring: the function waits (barrier) until no wave still reads the ring.
template <Epi EPI, int TM, int TN, int WTM, int WTN, typename Acc>
__device__ __forceinline__ void store_tile_staged(const Acc (&acc)[TN][TM], const float* __restrict__ s_tok,
                                                  const float* __restrict__ s_ch,
                                                  const uint16_t* __restrict__ bias, uint16_t* __restrict__ out,
                                                  int64_t M, int64_t N, int64_t mb, int64_t nb, int wm, int wn,
                                                  int frag_row, int frag_half, uint8_t* region, int lane) {
  constexpr int COLS = EPI == Epi::kSwiglu ? WTN / 2 : WTN;  // output columns of the wave's sub-tile
  constexpr int TNO = COLS / 32;                              // 32-column output blocks
  constexpr int ROWB = COLS * 2;                              // bytes per staged row
  constexpr int CPR = ROWB / 16;                              // 16-byte chunks per row
  static_assert(CPR == 4 || CPR == 8 || CPR == 16, "row of 4, 8 or 16 chunks");
  constexpr bool kPair = EPI == Epi::kSwiglu;
  const int64_t m0 = mb + (int64_t)wm * WTM, n0w = nb + (int64_t)wn * COLS;
  // Every scale and bias value the wave needs is loaded first and without
  // conditions, so that the wave waits for memory once: rows past M read row
  // M - 1, columns past N the last four (N is a multiple of 8 and a lane's
  // columns come in fours), and without a bias the loads read s_ch and are
  // replaced by zeros.  Such values only reach outputs that are never stored.
  // (Loads under per-element conditions were waited for one at a time: 24
  // round trips per wave at 192 x 128.)
  const bool has_bias = bias != nullptr;
  const uint16_t* bsrc = has_bias ? bias : reinterpret_cast<const uint16_t*>(s_ch);
  float st[TM];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) st[tm] = s_tok[min<int64_t>(m0 + tm * 32 + frag_row, M - 1)];
  float4 sg[TNO][4], su[kPair ? TNO : 1][4];
  uint2 bg_raw[TNO][4], bu_raw[kPair ? TNO : 1][4];
#pragma unroll
  for (int tn = 0; tn < TNO; ++tn)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t n = min<int64_t>(n0w + tn * 32 + 8 * q + 4 * frag_half, N - 4);
      sg[tn][q] = *reinterpret_cast<const float4*>(s_ch + n);
      bg_raw[tn][q] = *reinterpret_cast<const uint2*>(bsrc + n);
      if constexpr (kPair) {
        su[tn][q] = *reinterpret_cast<const float4*>(s_ch + N + n);
        bu_raw[tn][q] = *reinterpret_cast<const uint2*>(bsrc + N + n);
      }
    }
  lds_barrier();  // every wave is done with the operand ring
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int row = tm * 32 + frag_row;
#pragma unroll
    for (int tn = 0; tn < TNO; ++tn)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nl = tn * 32 + 8 * q + 4 * frag_half;  // column within the sub-tile
        float bg[4], y[4];
        bf16x4(has_bias ? bg_raw[tn][q] : make_uint2(0u, 0u), bg);
        const float sgv[4] = {sg[tn][q].x, sg[tn][q].y, sg[tn][q].z, sg[tn][q].w};
        if constexpr (!kPair) {
#pragma unroll
          for (int v = 0; v < 4; ++v) y[v] = __builtin_fmaf((float)acc[tn][tm][4 * q + v], st[tm] * sgv[v], bg[v]);
        } else {  // gate block tn, up block tn + TN/2
          float bu[4];
          bf16x4(has_bias ? bu_raw[tn][q] : make_uint2(0u, 0u), bu);
          const float suv[4] = {su[tn][q].x, su[tn][q].y, su[tn][q].z, su[tn][q].w};
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float g = __builtin_fmaf((float)acc[tn][tm][4 * q + v], st[tm] * sgv[v], bg[v]);
            const float u = __builtin_fmaf((float)acc[tn + TN / 2][tm][4 * q + v], st[tm] * suv[v], bu[v]);
            y[v] = silu_f32(g) * u;
          }
        }
        const uint2 hv = make_uint2(bf16x2_rne(y[0], y[1]), bf16x2_rne(y[2], y[3]));
        const int chunk = nl / 8;  // 16-byte chunk of the row; the lane's 8 bytes are its half frag_half
        *reinterpret_cast<uint2*>(region + row * ROWB + ((chunk ^ (row % CPR)) * 16) + 8 * frag_half) = hv;
      }
  }
  // (LDS accesses of one wave complete in order; the wave barrier keeps the
  // compiler from moving the reads above the writes)
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  constexpr int RPI = 64 / CPR;  // rows per store instruction
  const int c = lane % CPR;
#pragma unroll
  for (int r0 = 0; r0 < WTM; r0 += RPI) {
    const int row = r0 + lane / CPR;
    const int64_t m = m0 + row, n = n0w + c * 8;
    const u32x4 v = *reinterpret_cast<const u32x4*>(region + row * ROWB + ((c ^ (row % CPR)) * 16));
    // non-temporal: the output is not read again in this kernel, and lines
    // left dirty in the XCD's L2 would be written back at the kernel's end
    // (0.9 us of a 1502 x 4096 x 4096 launch)
    if (m < M && n < N) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(out + m * N + n));
  }
}

template <int BM, int BN, int WGM, int WGN, int BK, int NST, Epi EPI, bool FP8, bool PA, bool PB>
__global__ void __launch_bounds__(64 * WGM * WGN)
gemm_tile(const uint8_t* __restrict__ a, const float* __restrict__ s_tok,
          const uint8_t* __restrict__ b, const float* __restrict__ s_ch,
          const uint16_t* __restrict__ bias, void* __restrict__ out,
          int64_t M, int64_t N, int64_t K, int tiles_m, int tiles_n) {
  constexpr int NT = 64 * WGM * WGN;
  constexpr int CH = BK / 16;                       // 16-byte chunks per LDS row
  constexpr int NSUB = BK / 32;                     // 32-deep k substeps per stage
  constexpr int WTM = BM / WGM, WTN = BN / WGN;     // wave tile: tokens x weight rows
  constexpr int TM = WTM / 32, TN = WTN / 32;       // 32x32 MFMA blocks per wave
  constexpr int A_LOADS = BM * CH / NT, B_LOADS = BN * CH / NT;
  constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK, STAGE = A_BYTES + B_BYTES;
  constexpr int LOADS = A_LOADS + B_LOADS;          // per thread per stage
  static_assert(NSUB % 2 == 0 && NST >= 3, "even substeps per stage, three or more stages");
  static_assert(TM * 32 * WGM == BM && TN * 32 * WGN == BN, "wave tiles of 32x32 blocks");
  static_assert(A_LOADS * NT == BM * CH && B_LOADS * NT == BN * CH, "tile / threads");
  static_assert(!paired_epi(EPI) || TN % 2 == 0, "SwiGLU needs gate/up block pairs");
  static_assert(NST * LOADS < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NST * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % WGM, wn = wave / WGM;
  int tile_m, tile_n;
  tile_of_block(blockIdx.x, gridDim.x, tiles_m, tiles_n, tile_m, tile_n);
  const int64_t mb = (int64_t)tile_m * BM;
  // SwiGLU tiles cover BN/2 output columns: LDS weight rows [0, BN/2) are gate
  // rows, [BN/2, BN) the matching up rows.
  const int64_t nb = paired_epi(EPI) ? (int64_t)tile_n * (BN / 2) : (int64_t)tile_n * BN;

  // Direct-to-LDS loads: each wave instruction fills 64 consecutive 16-byte LDS
  // slots; slot p of a stage holds chunk (p % CH) ^ swizzle of tile row p / CH,
  // so each lane fetches the global chunk that belongs in its slot.  Offsets
  // are 32-bit and relative to a panel base that is uniform per load
  // instruction; rows past M (or past the weight's rows) re-read the last valid
  // row -- they only reach outputs never stored.  An operand is either
  // row-major [rows][K] or packed (PA / PB): blocks of 32 rows x 64 bytes,
  // block (r / 32, k / 64) at byte ((r / 32) * (K / 64) + k / 64) * 2048, so
  // that each 32-row, 64-byte piece of a stage is one contiguous 2 KiB read.
  // Panel bases are rows that are multiples of 32, at byte row * K in either
  // layout.
  auto src_off = [&](int64_t rel, int c, bool packed) -> uint32_t {
    if (packed)
      return (uint32_t)((rel / 32) * 32 * K + (rel % 32) * 64 + (c / 4) * 2048 + (c % 4) * 16);
    return (uint32_t)(rel * K + c * 16);
  };
  constexpr int ROWS_PER_LOAD = NT / CH;
  static_assert(!paired_epi(EPI) || (BN / 2) % ROWS_PER_LOAD == 0,
                "each load instruction reads gate rows only or up rows only");
  const uint8_t* a_panel = a + mb * K;
  // SwiGLU: gate rows nb.. and up rows N + nb..; the up panel starts at the
  // 32-row boundary at or below N + nb, so its relative rows start at up_skew.
  const int64_t up_first = N + nb;
  const int64_t up_base = PB ? up_first / 32 * 32 : up_first;
  const int64_t up_skew = up_first - up_base;
  const uint8_t* b_panel = b + nb * K;
  const uint8_t* b_up_panel = b + up_base * K;
  uint32_t a_off[A_LOADS], b_off[B_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) {
    const int p = i * NT + tid, r = p / CH, c = (p % CH) ^ swz_key<CH>(r);
    a_off[i] = src_off(min<int64_t>(r, M - 1 - mb), c, PA);
  }
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) {
    const int p = i * NT + tid, r = p / CH, c = (p % CH) ^ swz_key<CH>(r);
    if constexpr (paired_epi(EPI)) {
      const int64_t col = min<int64_t>(r % (BN / 2), N - 1 - nb);
      b_off[i] = src_off(r < BN / 2 ? col : up_skew + col, c, PB);
    } else {
      b_off[i] = src_off(min<int64_t>(r, N - 1 - nb), c, PB);
    }
  }
  // Stages past the last one re-load the last stage (their fragments, read by
  // the last stage, are never multiplied), so every stage issues the same
  // number of loads (constant vmcnt accounting, no branches in the loop body).
  const int64_t ksteps = K / BK;
  auto issue = [&](int64_t step) __attribute__((always_inline)) {
    // 32-bit per-stage offsets off a uniform panel base: the loads use the
    // scalar-base addressing form and keep one VGPR per load live, not two
    // (a stage of BK bytes advances BK bytes along a row-major row, or BK / 64
    // blocks of 2 KiB in the packed layout)
    const uint32_t ks = (uint32_t)min<int64_t>(step, ksteps - 1);
    const uint32_t ka = PA ? ks * (BK / 64) * 2048 : ks * BK;
    const uint32_t kb = PB ? ks * (BK / 64) * 2048 : ks * BK;
    uint8_t* st = lds + (int)(step % NST) * STAGE;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) lds_dma16(a_panel + (a_off[i] + ka), st + (i * NT + wave * 64) * 16);
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      const bool up = paired_epi(EPI) && i * ROWS_PER_LOAD >= BN / 2;  // compile-time per i
      lds_dma16((up ? b_up_panel : b_panel) + (b_off[i] + kb), st + A_BYTES + (i * NT + wave * 64) * 16);
    }
  };

  using Acc = typename std::conditional<FP8, v16f, v16i>::type;
  Acc acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = Acc{};

  // LDS rows this lane reads as MFMA operands: lane l supplies row l % 32 of a
  // 32-row block; lane half h = l / 32 supplies k bytes [32j + 16h, +16) of
  // substep j (for int8 one 32-deep MFMA; for E4M3FN two 16-deep bf16 MFMAs on
  // bytes [0, 8) and [8, 16) of those 16 -- the same k pairing for both
  // operands, which is all the dot product needs).
  const int frag_row = lane & 31, frag_half = lane >> 5;
  int a_rows[TM], b_rows[TN];
#pragma unroll
  for (int t = 0; t < TM; ++t) a_rows[t] = wm * WTM + t * 32 + frag_row;
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    if constexpr (paired_epi(EPI))
      b_rows[t] = (t < TN / 2 ? 0 : BN / 2) + wn * (WTN / 2) + (t % (TN / 2)) * 32 + frag_row;
    else
      b_rows[t] = wn * WTN + t * 32 + frag_row;
  }

  // Fragment register sets for two stages (set indices are compile-time
  // constants so the arrays stay in registers): a whole stage's fragments are
  // read from LDS one stage ahead of its MFMAs.  (Reading only one substep
  // ahead measured 1-2% slower on every workload.)
  v4i fa[2 * NSUB][TM], fb[2 * NSUB][TN];
  auto read_frags = [&](auto set_c, int64_t step, int sub) __attribute__((always_inline)) {
    constexpr int set = decltype(set_c)::value;
    const uint8_t* la = lds + (int)(step % NST) * STAGE;
    const uint8_t* lb = la + A_BYTES;
    const int c = 2 * sub + frag_half;
#pragma unroll
    for (int t = 0; t < TM; ++t) fa[set][t] = *reinterpret_cast<const v4i*>(la + swz<CH>(a_rows[t], c));
#pragma unroll
    for (int t = 0; t < TN; ++t) fb[set][t] = *reinterpret_cast<const v4i*>(lb + swz<CH>(b_rows[t], c));
  };
  auto mfmas = [&](auto set_c) __attribute__((always_inline)) {
    constexpr int set = decltype(set_c)::value;
    if constexpr (FP8) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        v8bf ca[TM];
#pragma unroll
        for (int t = 0; t < TM; ++t)
          ca[t] = e4m3x8_to_bf16(u32x2{(unsigned)fa[set][t][2 * j], (unsigned)fa[set][t][2 * j + 1]});
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const v8bf cb = e4m3x8_to_bf16(u32x2{(unsigned)fb[set][tn][2 * j], (unsigned)fb[set][tn][2 * j + 1]});
#pragma unroll
          for (int tm = 0; tm < TM; ++tm)
            acc[tn][tm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cb, ca[tm], acc[tn][tm], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
          acc[tn][tm] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[set][tn], fa[set][tm], acc[tn][tm], 0, 0, 0);
    }
  };

  // Stage s lives in LDS buffer s % NST; stages 0 .. NST-2 are issued up front.
  // Stage k's fragments are read during stage k - 1 (stage 0's after the
  // prologue).  At the start of stage k the wave waits until stage k + 1 has
  // landed (own loads: vmcnt) and the barrier makes that hold for every wave;
  // then stage k + NST - 1 is loaded into buffer (k - 1) % NST, the buffer of
  // stage k - 1, whose fragment reads every wave has completed (its MFMAs ran
  // before the barrier), and stage k + 1 is read while stage k is multiplied.
  // (Refilling the buffer of stage k instead needs an LDS-read drain before the
  // barrier: 6% slower at 192 x 128 on uniformly random codes, the same at
  // 256 x 256 and within 1% on the workloads' own data.)  Stages come in
  // pairs (K / BK even), so each stage's register sets are fixed at compile
  // time.  With one wave per SIMD any non-MFMA instruction between MFMAs idles
  // the matrix core, so LDS reads and loads are interleaved one per MFMA
  // (sched_group_barrier).
  constexpr int NMFMA = TM * TN * (FP8 ? 2 : 1);   // MFMAs per substep
  constexpr int NREAD = TM + TN;                    // ds_read_b128 per substep
  constexpr int RD_PER = (NREAD + NMFMA - 1) / NMFMA;            // LDS reads per MFMA slot
  constexpr int MEM_PER = (NREAD + LOADS + NMFMA - 1) / NMFMA;   // reads + loads per MFMA slot
#pragma unroll
  for (int s = 0; s < NST - 1; ++s) issue(s);
  wait_vmcnt<(NST - 2) * LOADS>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  static_for<0, NSUB>([&](auto j_c) __attribute__((always_inline)) {
    read_frags(std::integral_constant<int, decltype(j_c)::value>{}, 0, decltype(j_c)::value);
  });
  for (int64_t ks = 0; ks < ksteps; ks += 2) {
    static_for<0, 2>([&](auto p_c) __attribute__((always_inline)) {
      constexpr int p = decltype(p_c)::value;
      const int64_t k = ks + p;
      wait_vmcnt<(NST - 3) * LOADS>();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      static_for<0, NSUB>([&](auto j_c) __attribute__((always_inline)) {
        constexpr int j = decltype(j_c)::value;
        if constexpr (j == 0) issue(k + NST - 1);
        read_frags(std::integral_constant<int, (1 - p) * NSUB + j>{}, k + 1, j);
        mfmas(std::integral_constant<int, p * NSUB + j>{});
#pragma unroll
        for (int i = 0; i < NMFMA; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, j);  // one MFMA
          // LDS reads, plus in the first substep the stage's loads
          __builtin_amdgcn_sched_group_barrier(j == 0 ? 0x120 : 0x100, j == 0 ? MEM_PER : RD_PER, j);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    });
  }
  // the tail re-loads must land before the workgroup's LDS can be reused
  wait_vmcnt<0>();

  if constexpr (EPI == Epi::kRawI32) {
    store_tile_i32<TM, TN, WTM, WTN>(acc, static_cast<int32_t*>(out), M, N, mb, nb, wm, wn, frag_row, frag_half);
  } else {
    constexpr int REGION = WTM * (EPI == Epi::kSwiglu ? WTN / 2 : WTN) * 2;
    static_assert(REGION * WGM * WGN <= NST * STAGE, "staged output fits the operand ring");
    store_tile_staged<EPI, TM, TN, WTM, WTN>(acc, s_tok, s_ch, bias, static_cast<uint16_t*>(out), M, N, mb, nb,
                                             wm, wn, frag_row, frag_half, lds + wave * REGION, lane);
  }
}

template <int BM, int BN, int WGM, int WGN, int BK, int NST, Epi EPI, bool FP8, bool PA, bool PB>
hipError_t launch_cfg(const void* a, const float* s_tok, const void* b, const float* s_ch,
                      const uint16_t* bias, void* out, int64_t M, int64_t N, int64_t K,
                      hipStream_t stream) {
  const int64_t tiles_m = (M + BM - 1) / BM;
  const int64_t cols_per_tile = paired_epi(EPI) ? BN / 2 : BN;
  const int64_t tiles_n = (N + cols_per_tile - 1) / cols_per_tile;
  const int64_t blocks = tiles_m * tiles_n;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if ((K / BK) % 2 != 0) return hipErrorInvalidValue;  // stages come in pairs
  hipLaunchKernelGGL((gemm_tile<BM, BN, WGM, WGN, BK, NST, EPI, FP8, PA, PB>), dim3((unsigned)blocks),
                     dim3(64 * WGM * WGN), 0, stream, static_cast<const uint8_t*>(a), s_tok,
                     static_cast<const uint8_t*>(b), s_ch, bias, out, M, N, K, (int)tiles_m,
                     (int)tiles_n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Persistent form of the 256 x 256 tile (one workgroup per CU, walking the
// tiles of its XCD's range, P workgroups per XCD taking every P-th tile, so the
// tiles running at once on an XCD are the same as in a one-tile-per-workgroup
// launch).  Launched one tile per workgroup, every CU would finish its K loop
// at the same moment, write its output and then fetch the next tile's first
// stages, all CUs together: ~12 us per round of tiles measured at
// 12,016 x 5,120 x K (the intercept of the launch time against K).  Here the
// operand ring runs on from one tile into the next: the next tile's first
// stages are issued during this tile's last stages and land while its epilogue
// runs.  The epilogue therefore cannot stage its output in the ring: each wave
// stages 32 rows x half its columns at a time in an LDS area of its own, and
// the tile's token scales, channel scales and bias come into LDS by
// direct-to-LDS loads at the start of the tile (two areas, by tile parity, so
// the next tile's scales never overwrite ones a wave still reads).  Outputs go
// out as buffer stores, whose out-of-range lanes the hardware drops, so every
// wave issues the same number of stores and the vector-memory counts stay
// exact.  Wait counts (loads and stores complete in issue order): in the first
// two stages of every tile after the first, the epilogue's stores and the
// scale loads were issued after the stage being waited for.
typedef int i32x4 __attribute__((ext_vector_type(4)));

// 4 bytes per lane from global memory straight into LDS (lane i's at l + 4 i; l
// wave-uniform).
__device__ __forceinline__ void lds_dma4(const void* g, uint8_t* l) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, l, 4, 0, 0);
#endif
}

}  // namespace
}  // namespace w8a8
// 16 bytes per lane to a buffer (base and size in the wave-uniform resource; a lane
// whose offset is out of range stores nothing).
__device__ void w8a8_raw_buffer_store_x4(w8a8::i32x4 vdata, w8a8::i32x4 rsrc, int voffset, int soffset,
                                          int aux) __asm("llvm.amdgcn.raw.buffer.store.v4i32");
namespace w8a8 {
namespace {

constexpr uint32_t kOutOfRange = 0x80000000u;  // buffer offset past any persistent launch's output

template <Epi EPI, bool FP8, bool PA, bool PB>
__global__ void __launch_bounds__(256)
gemm_persist(const uint8_t* __restrict__ a, const float* __restrict__ s_tok,
             const uint8_t* __restrict__ b, const float* __restrict__ s_ch,
             const uint16_t* __restrict__ bias, void* __restrict__ out,
             int64_t M, int64_t N, int64_t K, int tiles_m, int tiles_n) {
  constexpr int BM = 256, BN = 256, WGM = 2, WGN = 2, BK = 64, NST = 4;
  constexpr int NT = 256;
  constexpr int CH = BK / 16;
  constexpr int NSUB = BK / 32;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int A_LOADS = BM * CH / NT, B_LOADS = BN * CH / NT;
  constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK, STAGE = A_BYTES + B_BYTES;
  constexpr int LOADS = A_LOADS + B_LOADS;
  constexpr bool kPair = paired_epi(EPI);
  constexpr bool kRaw = EPI == Epi::kRawI32;
  constexpr int COLS = kPair ? WTN / 2 : WTN;   // output columns of a wave's sub-tile
  constexpr int HALF = COLS / 2;                // columns staged at a time
  constexpr int TNO = COLS / 32, TNH = TNO / 2; // 32-column output blocks (per half)
  constexpr int ROWB = HALF * 2;                // bytes per staged row
  constexpr int CPR = ROWB / 16;                // 16-byte chunks per staged row
  constexpr int RPI = 64 / CPR;                 // staged rows per store instruction
  constexpr int SREG = 32 * ROWB;               // staging bytes per wave
  constexpr int RING = NST * STAGE;
  constexpr int SC_BYTES = 3 * 1024;            // s_tok[256] f32, s_ch[256] f32, bias 4 x 256 B
  constexpr int D = kRaw ? 0 : 3;                // scale / bias loads per wave per tile (the raw
                                                // int32 epilogue has no scales: its pointers are null)
  constexpr int S = kRaw ? 0 : TM * 2 * (32 / RPI);  // output stores per wave per tile (raw: counted as 0)
  constexpr int N0 = (NST - 3) * LOADS, N1 = N0 + S + D;
  static_assert(CPR == 4 || CPR == 8, "staged rows of 4 or 8 chunks");
  static_assert(N1 < 64, "vmcnt range");
  static_assert(!kPair || (BN / 2) % (NT / CH) == 0, "each load instruction reads gate rows only or up rows only");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[RING + 4 * SREG + 2 * SC_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WGM, wn = wave / WGM;
  const int frag_row = lane & 31, frag_half = lane >> 5;

  // this workgroup's tiles: XCD x's contiguous range, every per_xcd-th from idx
  const int ntiles = tiles_m * tiles_n;
  const int per_xcd = gridDim.x / kXcds;
  const int xcd = blockIdx.x % kXcds, idx = blockIdx.x / kXcds;
  const int q8 = ntiles / kXcds, r8 = ntiles % kXcds;
  const int t_first = xcd * q8 + min(xcd, r8);
  const int t_count = q8 + (xcd < r8 ? 1 : 0);
  if (idx >= t_count) return;
  const int64_t ksteps = K / BK;

  auto tile_mb = [&](int t) -> int64_t { int tm, tn; tile_coords(t, tiles_m, tiles_n, tm, tn); return (int64_t)tm * BM; };
  auto tile_nb = [&](int t) -> int64_t {
    int tm, tn; tile_coords(t, tiles_m, tiles_n, tm, tn);
    return kPair ? (int64_t)tn * (BN / 2) : (int64_t)tn * BN;
  };

  // ---- issue side: the tile and k of the next stage to load, its panels and offsets
  auto src_off = [&](int64_t rel, int c, bool packed) -> uint32_t {
    if (packed)
      return (uint32_t)((rel / 32) * 32 * K + (rel % 32) * 64 + (c / 4) * 2048 + (c % 4) * 16);
    return (uint32_t)(rel * K + c * 16);
  };
  constexpr int ROWS_PER_LOAD = NT / CH;
  int it_i = idx;                 // position of the issue tile in this XCD's range
  int64_t it_k = 0;               // next stage of the issue tile
  const uint8_t* a_panel;
  const uint8_t* b_panel;
  const uint8_t* b_up_panel;
  uint32_t a_off[A_LOADS], b_off[B_LOADS];
  auto set_issue_tile = [&](int t) __attribute__((always_inline)) {
    const int64_t mb = tile_mb(t), nb = tile_nb(t);
    a_panel = a + mb * K;
    const int64_t up_first = N + nb;
    const int64_t up_base = PB ? up_first / 32 * 32 : up_first;
    const int64_t up_skew = up_first - up_base;
    b_panel = b + nb * K;
    b_up_panel = b + up_base * K;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int p = i * NT + tid, r = p / CH, c = (p % CH) ^ swz_key<CH>(r);
      a_off[i] = src_off(min<int64_t>(r, M - 1 - mb), c, PA);
    }
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      const int p = i * NT + tid, r = p / CH, c = (p % CH) ^ swz_key<CH>(r);
      if constexpr (kPair) {
        const int64_t col = min<int64_t>(r % (BN / 2), N - 1 - nb);
        b_off[i] = src_off(r < BN / 2 ? col : up_skew + col, c, PB);
      } else {
        b_off[i] = src_off(min<int64_t>(r, N - 1 - nb), c, PB);
      }
    }
  };
  set_issue_tile(t_first + it_i);
  // Before each issue: past the issue tile's last stage move on to the next tile
  // of this workgroup; past the last tile keep re-loading its last stage (those
  // buffers are never multiplied; every stage issues the same loads).
  auto advance_issue = [&]() __attribute__((always_inline)) {
    if (it_k == ksteps) {
      if (it_i + per_xcd < t_count) {
        it_i += per_xcd;
        it_k = 0;
        set_issue_tile(t_first + it_i);
      } else {
        it_k = ksteps - 1;
      }
    }
  };
  int64_t g_issue = 0;  // global stage index of the next issue (ring buffer g % NST)
  auto issue = [&]() __attribute__((always_inline)) {
    const uint32_t ks = (uint32_t)it_k;
    const uint32_t ka = PA ? ks * (BK / 64) * 2048 : ks * BK;
    const uint32_t kb = PB ? ks * (BK / 64) * 2048 : ks * BK;
    uint8_t* st = lds + (int)(g_issue % NST) * STAGE;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) lds_dma16(a_panel + (a_off[i] + ka), st + (i * NT + wave * 64) * 16);
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      const bool up = kPair && i * ROWS_PER_LOAD >= BN / 2;
      lds_dma16((up ? b_up_panel : b_panel) + (b_off[i] + kb), st + A_BYTES + (i * NT + wave * 64) * 16);
    }
    ++g_issue;
    ++it_k;
  };

  // ---- scales and bias of a tile into LDS area (j & 1): wave w loads token rows
  // 64w.., channel columns 64w.. of the tile's 256 weight rows (gate rows then up
  // rows when paired), and bias pairs for those columns into its own 256-byte window
  const bool has_bias = bias != nullptr;
  auto load_scales = [&](int t, int j) __attribute__((always_inline)) {
    uint8_t* area = lds + RING + 4 * SREG + (j & 1) * SC_BYTES;
    const int64_t mb = tile_mb(t), nb = tile_nb(t);
    const int64_t m = min<int64_t>(mb + 64 * wave + lane, M - 1);
    lds_dma4(s_tok + m, area + wave * 256);
    const int c = 64 * wave + lane;  // local weight row of the tile
    int64_t n;
    if constexpr (kPair) n = c < BN / 2 ? min<int64_t>(nb + c, N - 1) : N + min<int64_t>(nb + c - BN / 2, N - 1);
    else n = min<int64_t>(nb + c, N - 1);
    lds_dma4(s_ch + n, area + 1024 + wave * 256);
    const int cp = 64 * wave + 2 * (lane & 31);  // first local row of the lane's bias pair
    int64_t nbp;
    if constexpr (kPair) nbp = cp < BN / 2 ? min<int64_t>(nb + cp, N - 2) : N + min<int64_t>(nb + cp - BN / 2, N - 2);
    else nbp = min<int64_t>(nb + cp, N - 2);
    const void* bsrc = has_bias ? static_cast<const void*>(bias + nbp) : static_cast<const void*>(s_ch + n);
    lds_dma4(bsrc, area + 2048 + wave * 256);
  };

  using Acc = typename std::conditional<FP8, v16f, v16i>::type;
  Acc acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int jj = 0; jj < TM; ++jj) acc[i][jj] = Acc{};

  int a_rows[TM], b_rows[TN];
#pragma unroll
  for (int t = 0; t < TM; ++t) a_rows[t] = wm * WTM + t * 32 + frag_row;
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    if constexpr (kPair)
      b_rows[t] = (t < TN / 2 ? 0 : BN / 2) + wn * (WTN / 2) + (t % (TN / 2)) * 32 + frag_row;
    else
      b_rows[t] = wn * WTN + t * 32 + frag_row;
  }
  v4i fa[2 * NSUB][TM], fb[2 * NSUB][TN];
  auto read_frags = [&](auto set_c, int64_t g, int sub) __attribute__((always_inline)) {
    constexpr int set = decltype(set_c)::value;
    const uint8_t* la = lds + (int)(g % NST) * STAGE;
    const uint8_t* lb = la + A_BYTES;
    const int c = 2 * sub + frag_half;
#pragma unroll
    for (int t = 0; t < TM; ++t) fa[set][t] = *reinterpret_cast<const v4i*>(la + swz<CH>(a_rows[t], c));
#pragma unroll
    for (int t = 0; t < TN; ++t) fb[set][t] = *reinterpret_cast<const v4i*>(lb + swz<CH>(b_rows[t], c));
  };
  auto mfmas = [&](auto set_c) __attribute__((always_inline)) {
    constexpr int set = decltype(set_c)::value;
    if constexpr (FP8) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        v8bf ca[TM];
#pragma unroll
        for (int t = 0; t < TM; ++t)
          ca[t] = e4m3x8_to_bf16(u32x2{(unsigned)fa[set][t][2 * jj], (unsigned)fa[set][t][2 * jj + 1]});
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const v8bf cb = e4m3x8_to_bf16(u32x2{(unsigned)fb[set][tn][2 * jj], (unsigned)fb[set][tn][2 * jj + 1]});
#pragma unroll
          for (int tm = 0; tm < TM; ++tm)
            acc[tn][tm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cb, ca[tm], acc[tn][tm], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
          acc[tn][tm] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[set][tn], fa[set][tm], acc[tn][tm], 0, 0, 0);
    }
  };

  // ---- the tile's epilogue (compute-side tile t, scale area j & 1)
  const i32x4 out_rsrc = {__builtin_amdgcn_readfirstlane((int)(uint32_t)reinterpret_cast<uint64_t>(out)),
                          __builtin_amdgcn_readfirstlane((int)(uint32_t)(reinterpret_cast<uint64_t>(out) >> 32)),
                          __builtin_amdgcn_readfirstlane((int)(uint32_t)(M * N * 2)), 0x00020000};
  auto epilogue = [&](int t, int j) __attribute__((always_inline)) {
    const int64_t mb = tile_mb(t), nb = tile_nb(t);
    if constexpr (kRaw) {
      store_tile_i32<TM, TN, WTM, WTN>(acc, static_cast<int32_t*>(out), M, N, mb, nb, wm, wn, frag_row, frag_half);
    } else {
      const uint8_t* area = lds + RING + 4 * SREG + (j & 1) * SC_BYTES;
      const float* st_l = reinterpret_cast<const float*>(area);
      const float* sc_l = reinterpret_cast<const float*>(area + 1024);
      const uint8_t* bi_l = area + 2048;
      uint8_t* region = lds + RING + wave * SREG;
      const int64_t m0 = mb + (int64_t)wm * WTM, n0w = nb + (int64_t)wn * COLS;
      const int lc0 = wn * COLS;  // the wave's first output column within the tile
      auto bias4 = [&](int lc, float* f) __attribute__((always_inline)) {  // local weight row lc, 4 values
        if (has_bias) bf16x4(*reinterpret_cast<const uint2*>(bi_l + (lc / 64) * 256 + (lc % 64) * 2), f);
        else f[0] = f[1] = f[2] = f[3] = 0.0f;
      };
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const float st = st_l[wm * WTM + tm * 32 + frag_row];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int tnh = 0; tnh < TNH; ++tnh) {
            const int tn = h * TNH + tnh;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int nl = tn * 32 + 8 * q + 4 * frag_half;  // column within the wave's sub-tile
              const int lc = lc0 + nl;
              const float4 sg = *reinterpret_cast<const float4*>(sc_l + lc);
              const float sgv[4] = {sg.x, sg.y, sg.z, sg.w};
              float bg[4], y[4];
              bias4(lc, bg);
              if constexpr (!kPair) {
#pragma unroll
                for (int v = 0; v < 4; ++v) y[v] = __builtin_fmaf((float)acc[tn][tm][4 * q + v], st * sgv[v], bg[v]);
              } else {
                const float4 su = *reinterpret_cast<const float4*>(sc_l + BN / 2 + lc);
                const float suv[4] = {su.x, su.y, su.z, su.w};
                float bu[4];
                bias4(BN / 2 + lc, bu);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                  const float gv = __builtin_fmaf((float)acc[tn][tm][4 * q + v], st * sgv[v], bg[v]);
                  const float uv = __builtin_fmaf((float)acc[tn + TN / 2][tm][4 * q + v], st * suv[v], bu[v]);
                  y[v] = silu_f32(gv) * uv;
                }
              }
              const uint2 hv = make_uint2(bf16x2_rne(y[0], y[1]), bf16x2_rne(y[2], y[3]));
              const int chunk = (nl - h * HALF) / 8;
              *reinterpret_cast<uint2*>(region + frag_row * ROWB + ((chunk ^ (frag_row % CPR)) * 16) + 8 * frag_half) = hv;
            }
          }
          __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
          __builtin_amdgcn_wave_barrier();
          const int c = lane % CPR;
#pragma unroll
          for (int r0 = 0; r0 < 32; r0 += RPI) {
            const int row = r0 + lane / CPR;
            const int64_t m = m0 + tm * 32 + row, n = n0w + h * HALF + c * 8;
            const u32x4 v = *reinterpret_cast<const u32x4*>(region + row * ROWB + ((c ^ (row % CPR)) * 16));
            const uint32_t off = (m < M && n < N) ? (uint32_t)((m * N + n) * 2) : kOutOfRange;
            w8a8_raw_buffer_store_x4(i32x4{(int)v.x, (int)v.y, (int)v.z, (int)v.w}, out_rsrc, (int)off, 0, 2);
          }
          __builtin_amdgcn_s_waitcnt(0xc07f);  // the reads are done before the region is rewritten
          __builtin_amdgcn_wave_barrier();
        }
      }
    }
  };

  constexpr int NMFMA = TM * TN * (FP8 ? 2 : 1);
  constexpr int NREAD = TM + TN;
  constexpr int RD_PER = (NREAD + NMFMA - 1) / NMFMA;
  constexpr int MEM_PER = (NREAD + LOADS + NMFMA - 1) / NMFMA;

  // prologue: the first tile's scales, then its first NST - 1 stages
  int j = 0;                 // tiles done by this workgroup
  int c_i = idx;             // position of the compute tile in this XCD's range
  if constexpr (!kRaw) load_scales(t_first + c_i, 0);
#pragma unroll
  for (int s = 0; s < NST - 1; ++s) { advance_issue(); issue(); }
  wait_vmcnt<(NST - 2) * LOADS>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  int64_t g = 0;  // global stage index being multiplied
  static_for<0, NSUB>([&](auto j_c) __attribute__((always_inline)) {
    read_frags(std::integral_constant<int, decltype(j_c)::value>{}, 0, decltype(j_c)::value);
  });
  while (true) {
    for (int64_t ks = 0; ks < ksteps; ks += 2) {
      const bool first_pair = ks == 0 && j > 0;
      static_for<0, 2>([&](auto p_c) __attribute__((always_inline)) {
        constexpr int p = decltype(p_c)::value;
        advance_issue();
        if (first_pair) wait_vmcnt<N1>();
        else wait_vmcnt<N0>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        static_for<0, NSUB>([&](auto j_c) __attribute__((always_inline)) {
          constexpr int jj = decltype(j_c)::value;
          if constexpr (jj == 0) issue();
          read_frags(std::integral_constant<int, (1 - p) * NSUB + jj>{}, g + 1, jj);
          mfmas(std::integral_constant<int, p * NSUB + jj>{});
#pragma unroll
          for (int i = 0; i < NMFMA; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, jj);
            __builtin_amdgcn_sched_group_barrier(jj == 0 ? 0x120 : 0x100, jj == 0 ? MEM_PER : RD_PER, jj);
          }
          __builtin_amdgcn_sched_barrier(0);
        });
        ++g;
      });
    }
    epilogue(t_first + c_i, j);
    ++j;
    c_i += per_xcd;
    if (c_i >= t_count) break;
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int jj = 0; jj < TM; ++jj) acc[i][jj] = Acc{};
    if constexpr (!kRaw) load_scales(t_first + c_i, j);
  }
  // every load into LDS has landed before the workgroup ends
  wait_vmcnt<0>();
}

template <Epi EPI, bool FP8, bool PA, bool PB>
hipError_t launch_persist(const void* a, const float* s_tok, const void* b, const float* s_ch,
                          const uint16_t* bias, void* out, int64_t M, int64_t N, int64_t K,
                          hipStream_t stream) {
  const int64_t tiles_m = (M + 255) / 256;
  const int64_t tiles_n = (N + (paired_epi(EPI) ? 127 : 255)) / (paired_epi(EPI) ? 128 : 256);
  const int64_t tiles = tiles_m * tiles_n;
  if ((K / 64) % 2 != 0 || K / 64 < 4 || tiles > 0x7fffffff) return hipErrorInvalidValue;
  const int64_t per_xcd = std::min<int64_t>((tiles + kXcds - 1) / kXcds, kCus / kXcds);
  hipLaunchKernelGGL((gemm_persist<EPI, FP8, PA, PB>), dim3((unsigned)(per_xcd * kXcds)), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(a), s_tok, static_cast<const uint8_t*>(b), s_ch, bias, out,
                     M, N, K, (int)tiles_m, (int)tiles_n);
  return hipGetLastError();
}

// Tile choice.  Candidates (all 4 waves, BK = 64, 4 stages):
//   256 x 256: waves of 128 x 128, 128 KiB LDS, one workgroup per CU;
//   192 x 128: waves of  96 x  64,  80 KiB LDS, two per CU;
//   128 x 128: waves of  64 x  64,  64 KiB LDS, two per CU.
// The kernel is throughput-bound per CU, so the time of a launch is taken as
// (tiles per CU, rounded up) x (tile area) / (relative efficiency of the tile
// shape); the efficiencies are the ops per CU-second of each shape relative to
// 256 x 256, measured on 12,016 x 5,120 x 17,408 (0.90 and 0.80).  Ties go to
// the larger tile.
template <Epi EPI, bool FP8, bool PA, bool PB>
hipError_t launch_t(const void* a, const float* s_tok, const void* b, const float* s_ch,
                    const uint16_t* bias, void* out, int64_t M, int64_t N, int64_t K,
                    hipStream_t stream) {
  const int64_t nw = paired_epi(EPI) ? 2 * N : N;  // weight rows
  auto cost = [&](int bm, int bn, double eff) {
    const int64_t tiles = ((M + bm - 1) / bm) * ((nw + bn - 1) / bn);
    return (double)((tiles + kCus - 1) / kCus) * bm * bn / eff;
  };
  const double c256 = cost(256, 256, 1.0), c192 = cost(192, 128, 0.90), c128 = cost(128, 128, 0.80);
  if (c256 <= c192 && c256 <= c128) {
    // persistent form: at least four stages per tile (the scale loads of a tile are
    // waited for by its third stage) and an output a 31-bit buffer offset reaches
    const int64_t out_bytes = M * N * (EPI == Epi::kRawI32 ? 4 : 2);
    if (K / 64 >= 4 && out_bytes < (int64_t)kOutOfRange)
      return launch_persist<EPI, FP8, PA, PB>(a, s_tok, b, s_ch, bias, out, M, N, K, stream);
    return launch_cfg<256, 256, 2, 2, 64, 4, EPI, FP8, PA, PB>(a, s_tok, b, s_ch, bias, out, M, N, K, stream);
  }
  if (c192 <= c128)
    return launch_cfg<192, 128, 2, 2, 64, 4, EPI, FP8, PA, PB>(a, s_tok, b, s_ch, bias, out, M, N, K, stream);
  return launch_cfg<128, 128, 2, 2, 64, 4, EPI, FP8, PA, PB>(a, s_tok, b, s_ch, bias, out, M, N, K, stream);
}

template <Epi EPI, bool FP8>
hipError_t launch_layouts(bool pa, bool pb, const void* a, const float* s_tok, const void* b,
                          const float* s_ch, const uint16_t* bias, void* out, int64_t M, int64_t N,
                          int64_t K, hipStream_t stream) {
  if (!pa && !pb) return launch_t<EPI, FP8, false, false>(a, s_tok, b, s_ch, bias, out, M, N, K, stream);
  if (pa && !pb) return launch_t<EPI, FP8, true, false>(a, s_tok, b, s_ch, bias, out, M, N, K, stream);
  if (pa && pb) return launch_t<EPI, FP8, true, true>(a, s_tok, b, s_ch, bias, out, M, N, K, stream);
  return hipErrorInvalidValue;
}

// Row-major [rows][K] -> packed blocks of 32 rows x 64 bytes (rows past `rows`
// in the last block are zero).  One thread per 16 destination bytes, so the
// writes are contiguous.
__global__ void __launch_bounds__(256)
pack_rows_kernel(const uint8_t* __restrict__ src, int64_t rows, int64_t K, uint8_t* __restrict__ dst,
                 int64_t chunks) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= chunks) return;
  const int64_t d = j * 16;
  const int64_t block = d / 2048, within = d % 2048;
  const int64_t kblocks = K / 64;
  const int64_t row = (block / kblocks) * 32 + within / 64;
  const int64_t k = (block % kblocks) * 64 + within % 64;
  u32x4 v = u32x4{0, 0, 0, 0};
  if (row < rows) v = *reinterpret_cast<const u32x4*>(src + row * K + k);
  *reinterpret_cast<u32x4*>(dst + d) = v;
}

}  // namespace

hipError_t launch_gemm(Epi epi, bool fp8, bool packed_a, bool packed_b, const void* a,
                       const float* s_tok, const void* b, const float* s_ch, const uint16_t* bias,
                       void* out, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  if (fp8) {
    if (epi == Epi::kDequant)
      return launch_layouts<Epi::kDequant, true>(packed_a, packed_b, a, s_tok, b, s_ch, bias, out, M, N, K, stream);
    return hipErrorInvalidValue;
  }
  switch (epi) {
    case Epi::kRawI32:
      return launch_layouts<Epi::kRawI32, false>(packed_a, packed_b, a, s_tok, b, s_ch, bias, out, M, N, K, stream);
    case Epi::kDequant:
      return launch_layouts<Epi::kDequant, false>(packed_a, packed_b, a, s_tok, b, s_ch, bias, out, M, N, K, stream);
    case Epi::kSwiglu:
      return launch_layouts<Epi::kSwiglu, false>(packed_a, packed_b, a, s_tok, b, s_ch, bias, out, M, N, K, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_pack_rows(const void* src, int64_t rows, int64_t K, void* dst, hipStream_t stream) {
  const int64_t chunks = packed_rows(rows) * K / 16;
  const int64_t blocks = (chunks + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(src), rows, K, static_cast<uint8_t*>(dst), chunks);
  return hipGetLastError();
}

}  // namespace w8a8
