// gemm_expert.hip -- expert projections over many rows per expert (prefill).
//
// The gate/up projection with SwiGLU (step A5) and the down projection
// (step A6) of every route row against its expert's MXFP4 weights, W4A16:
// "Muse Spark Open on Gaudi 2", section "What was built" (experts run W4A16)
// and section "The latent MoE: A' with a per-expert norm" (one row per
// (token, route) pair, the cost paid per touched expert slice).
//
// Workgroup tile: 128 route rows of one expert x 256 weight rows, eight
// wavefronts in a 2 x 4 grid, each computing 64 x 64 (4 x 4 fragments of bf16
// MFMA 16x16x32, fp32 accumulation); NVFP4 in a 1 x 8 grid, each wavefront
// 128 x 32 (8 x 2 fragments), so that each weight fragment is decoded once. Per stage of 64 reduction elements the
// activation rows (bf16, gathered through the grouping's route order) and
// the weight codes (4 bits per element, as stored) are copied straight from
// global memory into LDS by buffer loads with the LDS destination, in a ring
// of two stages, so the copies of the next stage run under the MFMAs. The E8M0
// scales of the tile's weight rows (K/32 bytes per row) are copied into LDS
// once. Each wavefront decodes its weight fragments from LDS with the gfx950
// scaled FP4 -> bf16 conversion just before its MFMAs: no bf16 copy of a
// weight exists anywhere. NVFP4 weights (one E4M3 scale per 16 elements,
// K/16 bytes per row) do not fit resident: their scales follow in blocks of
// 32 bytes per row (8 stages), double-buffered, each copied at the start of
// the block before it; the per-tensor fp32 scale multiplies the sums.
//
// LDS layouts (all conflict-free for the reads below):
//  - activations: 128-byte rows, 16-byte piece c of row r at position
//    r*8 + (c ^ ((r/2) % 8));
//  - weight codes: 32-byte rows, 16-byte piece p of row r at position
//    r*2 + (p ^ ((r/8) % 2));
//  - scales: K/32 bytes per row, 16-byte piece j of row r at position
//    j ^ ((r/2) & m) within the row, m + 1 the largest power of two dividing
//    the row's piece count (8 at K = 4096; the 16 rows a quarter-wave
//    reads at one offset then fall on 16 different 8-byte bank pairs; row-
//    major they fell on two); NVFP4: 32 bytes per row and block of 8 stages,
//    two blocks, row-major.
//
// Reduction order inside a 32-element block: lane group g = lane/16 owns
// elements 8g .. 8g+7 for both operands (its 4 code bytes and the block's
// scale byte). A tile's rows are split between the wavefront rows; a
// wavefront runs the MFMAs of its first 8 (NVFP4), 4, 2, 1 or 0 fragments of
// 16 rows (chosen once per tile, so the inner loop has no branches) and
// always takes its share of the copies.
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kEW = 8;                    // wavefronts per workgroup (2 x 4)
// Row tiles dealt to the XCDs in pairs (with their column tiles): an
// expert's full tile and its partial tail, side by side in the tile list,
// then run on one XCD and share its weight stream there (with single row
// tiles, 130 rows per expert ran 3.37 ms for gate/up, alternating full tiles
// and 2-row tails over the XCDs; in pairs 2.60 ms, real routing unchanged).
constexpr int kEChunk = 2;
constexpr int kEM = kExpertTileRows;      // tile rows (128)
constexpr int kEN = 256;                  // weight rows per tile
constexpr int kEK = 64;                   // reduction elements per stage
// Two stages in LDS (the copies of stage s + 1 run under the MFMAs of stage
// s) and the scales of K <= 4096 keep a workgroup at 80 KiB of LDS and under
// 128 VGPRs, so two workgroups share a compute unit; deeper rings raise the
// register count past that and measured slower.
constexpr int kERing = 2;                 // stages held in LDS (copies run kERing - 1 ahead)
constexpr int kEKMax = 4096;              // largest K (scales resident in LDS)
constexpr int kEAOps = kEM * kEK * 2 / 1024 / kEW;   // 1-KiB activation copies per wavefront and stage (2)
constexpr int kEBOps = kEN * kEK / 2 / 1024 / kEW;   // 1-KiB code copies per wavefront and stage (1)
constexpr int kEOps = kEAOps + kEBOps;
static_assert(kEM == 128, "two wavefront rows of 64");
// Light tiles (at most 16 rows): the two ring slots' LDS, 48 KiB, re-cut into
// kELRing slots of 16 activation rows (2 KiB, in the codes' array) and the
// tile's codes (8 KiB, in the activations' array), so that copies run three
// stages ahead instead of one: such a tile streams its weights with little
// MFMA work, and with one stage ahead its workgroup kept only about 9 KiB of
// HBM reads in flight.
constexpr int kELRows = 16;
constexpr int kELRing = 4;
constexpr int kELA = kELRows * kEK * 2;  // activation bytes per light slot
constexpr int kELB = kEN * kEK / 2;      // code bytes per light slot
static_assert(kELRing * kELA <= kERing * kEN * kEK / 2 && kELRing * kELB <= kERing * kEM * kEK * 2,
              "light slots fit the ring");
static_assert(kELRows == 2 * 8 && kEAOps == 2, "wavefront 0's two activation copies hold the 16 rows");

__device__ __forceinline__ int apos(int r, int c) { return (r * 8 + (c ^ ((r >> 1) & 7))) * 8; }
__device__ __forceinline__ int bpos(int r, int p) { return (r * 2 + (p ^ ((r >> 3) & 1))) * 16; }

template <int BFMT, int EPI>
__global__ __launch_bounds__(64 * kEW) void expert_kernel(TiledArgs p) {
  constexpr bool NV = BFMT == B_NVFP4;
  // Wavefront grid: MXFP4 2 x 4 (64 rows x 64 weight rows each); NVFP4,
  // whose decode (a multiply per weight) costs more than the MFMAs it
  // feeds, 1 x 8 (all 128 rows x 32 weight rows), so that each weight
  // fragment is decoded once per workgroup instead of once per wavefront
  // row, for twice the activation reads from LDS.
  constexpr int kWR = NV ? 1 : 2;       // wavefront rows
  constexpr int kMF = 4 * 2 / kWR;      // 16-row fragments per wavefront
  constexpr int kNF = 4 * kWR / 2;      // 16-column weight fragments per wavefront
  constexpr int kSsBytes = NV ? 2 * kEN * 32 : kEN * (kEKMax / 32);
  __shared__ __attribute__((aligned(1024))) uint16_t As[kERing][kEM * kEK];      // 16 KiB per stage
  __shared__ __attribute__((aligned(1024))) uint8_t Bs[kERing][kEN * kEK / 2];   // 8 KiB per stage
  __shared__ __attribute__((aligned(1024))) uint8_t Ss[kSsBytes];                // 32 KiB (NVFP4 16 KiB)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nl = lane & 15, g = lane >> 4;
  const int wm = kWR == 2 ? (wave & 1) : 0, wn = kWR == 2 ? (wave >> 1) : wave;

  // ---- XCD-aware tile order: two row tiles' column tiles on one XCD ----
  const int logical = xcd_tile(kEChunk * p.n_col_tiles);
  const int mt = logical / p.n_col_tiles, nt = logical % p.n_col_tiles;
  if (mt >= p.counters[1]) return;
  const int expert = p.tiles[2 * mt];
  const int row_begin = p.tiles[2 * mt + 1];
  // (a tile list no grouping of this call has written is skipped)
  if (expert < 0 || expert >= p.n_experts || row_begin < 0 || row_begin >= p.n_routes) return;
  const int row_end = min(row_begin + kEM, min(p.offsets[expert + 1], p.n_routes));
  if (row_end <= row_begin) return;
  // (the split into light and heavy experts: a light one is the streaming kernel's)
  if (p.offsets[expert + 1] - p.offsets[expert] <= p.min_rows) return;
  const int nrows = row_end - row_begin;  // >= 1
  const uint32_t K = static_cast<uint32_t>(p.K);

  // weight row of tile-local row r (r = wn*16*kNF + f*16 + nl)
  auto weight_row = [&](int r) -> int {
    const int w = r / (16 * kNF), f = (r >> 4) % kNF, n = r & 15;
    // fragments [0, kNF/2): gate rows; [kNF/2, kNF): the matching up rows
    if (EPI == EPI_SWIGLU)
      return (f / (kNF / 2)) * p.inter + nt * (kEN / 2) + w * (8 * kNF) + (f % (kNF / 2)) * 16 + n;
    return nt * kEN + r;
  };

  const size_t rows = static_cast<size_t>(p.b_rows_per_expert);
  const rsrc_t bq_r = make_rsrc(p.b_codes + expert * rows * (K / 2), static_cast<uint32_t>(rows * (K / 2)));
  constexpr int SB = NV ? 16 : 32;  // elements per scale byte
  const rsrc_t bs_r = make_rsrc(p.b_scales + expert * rows * (K / SB), static_cast<uint32_t>(rows * (K / SB)));
  const rsrc_t a_r = make_rsrc(p.a, p.a_bytes);

  // ---- source offsets of this wavefront's copies ----
  uint32_t aoff[kEAOps], boff[kEBOps];
#pragma unroll
  for (int i = 0; i < kEAOps; ++i) {
    const int r = (kEAOps * wave + i) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    aoff[i] = kOutOfRange;
    if (r < nrows) {
      const int pos = row_begin + r;
      const int ar = p.a_gather ? p.sorted[pos] / p.topk : pos;
      aoff[i] = static_cast<uint32_t>(ar) * K * 2 + c * 16;
    }
  }
#pragma unroll
  for (int i = 0; i < kEBOps; ++i) {
    const int r = (kEBOps * wave + i) * 32 + (lane >> 1);
    const int pc = (lane & 1) ^ ((r >> 3) & 1);
    boff[i] = static_cast<uint32_t>(weight_row(r)) * (K / 2) + pc * 16;
  }
  const uint32_t lds_a = static_cast<uint32_t>(reinterpret_cast<size_t>(
      (__attribute__((address_space(3))) uint16_t*)(&As[0][0])));
  const uint32_t lds_b = static_cast<uint32_t>(reinterpret_cast<size_t>(
      (__attribute__((address_space(3))) uint8_t*)(&Bs[0][0])));
  const uint32_t lds_s = static_cast<uint32_t>(reinterpret_cast<size_t>(
      (__attribute__((address_space(3))) uint8_t*)(&Ss[0])));

  auto issue = [&](int st, int slot, auto light_tag) __attribute__((always_inline)) {
    if constexpr (decltype(light_tag)::value) {  // (rows 0..15 are wavefront 0's two copies)
      if (wave == 0) {
#pragma unroll
        for (int i = 0; i < kEAOps; ++i)
          lds_copy16(a_r, aoff[i] + st * (kEK * 2), __builtin_amdgcn_readfirstlane(lds_b + slot * kELA + i * 1024));
      }
      lds_copy16(bq_r, boff[0] + st * (kEK / 2), __builtin_amdgcn_readfirstlane(lds_a + slot * kELB + wave * 1024));
      return;
    }
#pragma unroll
    for (int i = 0; i < kEAOps; ++i)
      lds_copy16(a_r, aoff[i] + st * (kEK * 2),
                 __builtin_amdgcn_readfirstlane(lds_a + slot * (kEM * kEK * 2) + (kEAOps * wave + i) * 1024));
#pragma unroll
    for (int i = 0; i < kEBOps; ++i)
      lds_copy16(bq_r, boff[i] + st * (kEK / 2),
                 __builtin_amdgcn_readfirstlane(lds_b + slot * (kEN * kEK / 2) + (kEBOps * wave + i) * 1024));
  };

  // ---- scales of the tile's weight rows ----
  // MXFP4: K/32 bytes per row, 16-byte pieces, copied once. NVFP4: one
  // 8-stage block (32 bytes per row) per wavefront copy, rows 32w .. 32w+31.
  const uint32_t s_src = NV ? static_cast<uint32_t>(weight_row(wave * 32 + (lane >> 1))) * (K / 16) +
                                  (lane & 1) * 16
                            : 0u;
  auto issue_scales = [&](int blk, int half) __attribute__((always_inline)) {
    lds_copy16(bs_r, s_src + blk * 32,
               __builtin_amdgcn_readfirstlane(lds_s + half * (kEN * 32) + wave * 1024));
  };
  const int spr = static_cast<int>(K / 512);  // MXFP4: 16-byte scale pieces per row
  // (the XOR stays inside an aligned block of pieces: the largest power of
  // two dividing the piece count)
  const int smask = (spr & -spr) - 1;
  if constexpr (!NV) {
    const int sblocks = kEN * spr / 64;         // 1-KiB blocks (K / 128)
    for (int q = wave; q < sblocks; q += kEW) {
      const int piece = q * 64 + lane;
      const int r = piece / spr, j = piece - r * spr;  // (LDS position j of row r holds piece j ^ swz)
      lds_copy16(bs_r, static_cast<uint32_t>(weight_row(r)) * (K / 32) + (j ^ ((r >> 1) & smask)) * 16,
                 __builtin_amdgcn_readfirstlane(lds_s + q * 1024));
    }
  }

  f32x4 acc[kMF][kNF];
#pragma unroll
  for (int m = 0; m < kMF; ++m)
#pragma unroll
    for (int f = 0; f < kNF; ++f) acc[m][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  // scale bytes of this lane's weight rows (one per fragment) for 8
  // consecutive 32-element blocks (4 stages), read from LDS once per 4
  // stages (NVFP4: 16 bytes, two per 32-element block)
  uint2 sreg[kNF];
  uint4 sreg4[kNF];
  // (the rows' swizzle, (r/2) & smask, is the same for a lane's four
  // fragments: they and the wavefront's rows start at multiples of 16)
  const int sx = (nl >> 1) & smask;
  auto read_scales = [&](int st) __attribute__((always_inline)) {
    const int soff = (((st >> 3) ^ sx) << 4) + (st & 7) * 2;
#pragma unroll
    for (int f = 0; f < kNF; ++f) {
      const int r = wn * 16 * kNF + f * 16 + nl;
      if constexpr (NV)
        sreg4[f] = *reinterpret_cast<const uint4*>(&Ss[((st / 8) & 1) * (kEN * 32) + r * 32 + (st % 8) * 4]);
      else  // (stages st .. st+3: bytes 2st .. 2st+7 of the row, in piece st/8)
        sreg[f] = *reinterpret_cast<const uint2*>(&Ss[r * (K / 32) + soff]);
    }
  };

  // MFMAs of one stage (q = stage mod 4) for the first LIVE fragments of
  // this wavefront's rows
  auto compute = [&](int slot, auto q_tag, auto live_tag, auto light_tag) __attribute__((always_inline)) {
    constexpr int LIVE = decltype(live_tag)::value;
    constexpr int q = decltype(q_tag)::value;
    constexpr bool LIGHT = decltype(light_tag)::value;
    if constexpr (LIVE == 0) {
      return;
    } else {
      const uint16_t* as = LIGHT ? reinterpret_cast<const uint16_t*>(&Bs[0][0] + slot * kELA) : As[slot];
      const uint8_t* bs = LIGHT ? reinterpret_cast<const uint8_t*>(&As[0][0]) + slot * kELB : Bs[slot];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int kb = q * 2 + s;  // block within the 8 held in sreg
        bf16x8 bv[kNF];
#pragma unroll
        for (int f = 0; f < kNF; ++f) {
          const int r = wn * 16 * kNF + f * 16 + nl;
          const uint32_t d = *reinterpret_cast<const uint32_t*>(&bs[bpos(r, s) + g * 4]);
          if constexpr (NV) {
            // block kb's two E4M3 bytes are 2kb, 2kb+1 of the 16; lane group g's
            // eight elements lie in the first 16 for g < 2
            const uint4 q4 = sreg4[f];
            const uint32_t w = (kb >> 1) == 0 ? q4.x : (kb >> 1) == 1 ? q4.y : (kb >> 1) == 2 ? q4.z : q4.w;
            bv[f] = nvfp4x8_to_bf16(d, e4m3_to_f32((w >> (16 * (kb & 1) + 8 * (g >> 1))) & 0xFFu));
          } else {
            const uint32_t w = kb < 4 ? sreg[f].x : sreg[f].y;
            bv[f] = mxfp4x8_to_bf16(d, e8m0_to_f32((w >> (8 * (kb & 3))) & 0xFFu));
          }
        }
        bf16x8 av[LIVE];
#pragma unroll
        for (int m = 0; m < LIVE; ++m)
          av[m] = as_bf16x8(*reinterpret_cast<const uint4*>(&as[apos(wm * 64 + m * 16 + nl, s * 4 + g)]));
#pragma unroll
        for (int m = 0; m < LIVE; ++m)
#pragma unroll
          for (int f = 0; f < kNF; ++f) acc[m][f] = mfma16x16x32(av[m], bv[f], acc[m][f]);
      }
    }
  };

  // Stage s lives in slot s % kERing. Copies past the last stage repeat it
  // into a slot that is no longer read, so the loop has no conditional
  // loads. The stage count (K / 64) is a multiple of 8.
  const int nst = static_cast<int>(K) / kEK;
  const int nblk = nst / 8;  // NVFP4 scale blocks
  auto kloop = [&](auto live_tag, auto light_tag) __attribute__((always_inline)) {
    constexpr bool LIGHT = decltype(light_tag)::value;
    constexpr int R = LIGHT ? kELRing : kERing;  // slots; copies run R - 1 stages ahead
    // until stage st + 1 has landed, the copies of the R - 2 stages after it
    // may be outstanding (light: wavefront 0 issues three copies per stage,
    // the others one)
    auto wait_next = [&]() __attribute__((always_inline)) {
      if constexpr (LIGHT) {
        if (wave == 0)
          wait_vm_keep<(kEAOps + 1) * (R - 2)>();
        else
          wait_vm_keep<R - 2>();
      } else {
        wait_vm_keep<kEOps * (R - 2)>();
      }
    };
    if constexpr (NV) issue_scales(0, 0);
#pragma unroll
    for (int s = 0; s < R - 1; ++s) issue(min(s, nst - 1), s, light_tag);
    wait_next();  // the scales and stage 0
    __syncthreads();
    int slot = 0;
    auto one = [&](int st, auto q_tag) __attribute__((always_inline)) {
      const int ahead = slot == 0 ? R - 1 : slot - 1;  // (st + R - 1) % R
      // (NVFP4: the next scale block goes out first, so this stage's wait,
      // which takes every copy issued before this stage's own, covers it)
      if constexpr (NV)
        if (decltype(q_tag)::value == 0 && st % 8 == 0)
          issue_scales(min(st / 8 + 1, nblk - 1), (st / 8 + 1) & 1);
      issue(min(st + R - 1, nst - 1), ahead, light_tag);
      compute(slot, q_tag, live_tag, light_tag);
      wait_next();  // stage st + 1 has landed
      __syncthreads();
      slot = slot == R - 1 ? 0 : slot + 1;
    };
    for (int st = 0; st < nst; st += 4) {
      if (decltype(live_tag)::value > 0) read_scales(st);
      one(st, std::integral_constant<int, 0>{});
      one(st + 1, std::integral_constant<int, 1>{});
      one(st + 2, std::integral_constant<int, 2>{});
      one(st + 3, std::integral_constant<int, 3>{});
    }
    wait_vm_keep<0>();  // no copy may still target this workgroup's LDS
  };
  const int wrows = min(max(nrows - wm * 64, 0), 16 * kMF);
  const int live = (wrows + 15) / 16;
  constexpr std::false_type kFull{};
  constexpr std::true_type kLight{};
  if (nrows <= kELRows) {  // (the same for every wavefront of the workgroup)
    if (live > 0)
      kloop(std::integral_constant<int, 1>{}, kLight);
    else
      kloop(std::integral_constant<int, 0>{}, kLight);
  } else if (kMF == 8 && live > 4) {
    kloop(std::integral_constant<int, kMF>{}, kFull);
  } else if (live > 2) {
    kloop(std::integral_constant<int, 4>{}, kFull);
  } else if (live > 1) {
    kloop(std::integral_constant<int, 2>{}, kFull);
  } else if (live > 0) {
    kloop(std::integral_constant<int, 1>{}, kFull);
  } else {
    kloop(std::integral_constant<int, 0>{}, kFull);
  }

  // ---- epilogue ----
  const float gs = NV ? p.b_global[expert] : 1.0f;
#pragma unroll
  for (int m = 0; m < kMF; ++m) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 64 + m * 16 + 4 * g + i;
      if (r >= nrows) continue;
      const int pos = row_begin + r;
      if (EPI == EPI_SWIGLU) {
        const int col = nt * (kEN / 2) + wn * (8 * kNF) + nl;
#pragma unroll
        for (int f = 0; f < kNF / 2; ++f) {
          const float gt = acc[m][f][i] * gs, up = acc[m][f + kNF / 2][i] * gs;
          const float silu = gt / (1.0f + expf(-gt));
          static_cast<uint16_t*>(p.out)[static_cast<size_t>(pos) * p.ldo + col + f * 16] = f32_to_bf16(silu * up);
        }
      } else {
        float* dst = static_cast<float*>(p.out) + static_cast<size_t>(p.sorted[pos]) * p.ldo + nt * kEN +
                     wn * 16 * kNF + nl;
#pragma unroll
        for (int f = 0; f < kNF; ++f) dst[f * 16] = acc[m][f][i] * gs;
      }
    }
  }
}

template <int EPI>
hipError_t launch_expert(const TiledArgs& a, int n_row_tiles, bool nvfp4, hipStream_t st) {
  const int n = n_row_tiles * a.n_col_tiles;
  const dim3 grid(xcd_grid(n, kEChunk * a.n_col_tiles)), block(64 * kEW);
  if (nvfp4)
    MOE_LAUNCH((expert_kernel<B_NVFP4, EPI>), grid, block, 0, st, a);
  else
    MOE_LAUNCH((expert_kernel<B_MXFP4, EPI>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace

int expert_chunk_rows() { return kEChunk; }

bool expert_lds_ok(int latent, int inter, bool nvfp4) {
  // K a multiple of 512 (whole 16-byte MXFP4 scale pieces per row, whole
  // 8-stage NVFP4 scale blocks); MXFP4 scales resident: K at most kEKMax
  if (latent % 512 || inter % 512) return false;
  return nvfp4 || (latent <= kEKMax && inter <= kEKMax);
}

hipError_t launch_gateup_expert(const ExpertGemm& x, hipStream_t st) {
  TiledArgs p{};
  p.grouped = 1;
  p.a = x.lat;
  p.a_bytes = static_cast<uint32_t>(static_cast<size_t>(x.tokens) * x.latent * 2);
  p.a_gather = 1;
  p.sorted = x.sorted;
  p.topk = x.topk;
  p.offsets = x.offsets;
  p.counters = x.counters;
  p.tiles = x.tiles;
  p.b_codes = x.w13_codes;
  p.b_scales = x.w13_scales;
  p.b_global = x.w13_global;
  p.n_experts = x.n_experts;
  p.n_routes = x.tokens * x.topk;
  p.b_rows_per_expert = 2 * x.inter;
  p.K = x.latent;
  p.inter = x.inter;
  p.out = x.h;
  p.ldo = x.inter;
  p.n_col_tiles = x.inter / (kEN / 2);
  p.min_rows = x.split_rows;
  return launch_expert<EPI_SWIGLU>(p, x.max_tiles, x.nvfp4, st);
}

hipError_t launch_down_expert(const ExpertGemm& x, hipStream_t st) {
  TiledArgs p{};
  p.grouped = 1;
  p.a = x.h;
  p.a_bytes = static_cast<uint32_t>(static_cast<size_t>(x.tokens) * x.topk * x.inter * 2);
  p.a_gather = 0;
  p.sorted = x.sorted;
  p.topk = x.topk;
  p.offsets = x.offsets;
  p.counters = x.counters;
  p.tiles = x.tiles;
  p.b_codes = x.w2_codes;
  p.b_scales = x.w2_scales;
  p.b_global = x.w2_global;
  p.n_experts = x.n_experts;
  p.n_routes = x.tokens * x.topk;
  p.b_rows_per_expert = x.latent;
  p.K = x.inter;
  p.out = x.rows;
  p.ldo = x.latent;
  p.n_col_tiles = x.latent / kEN;
  p.min_rows = x.split_rows;
  return launch_expert<EPI_F32_SCATTER>(p, x.max_tiles, x.nvfp4, st);
}

}  // namespace moe
