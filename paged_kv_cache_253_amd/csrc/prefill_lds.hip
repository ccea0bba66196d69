// Chunked prefill with long query runs ("vLLM & High-Throughput Serving",
// section 4): the wavefronts of a workgroup share each 32-token step's K
// and V tiles through LDS (the per-column work is that of prefill_mfma.hip,
// prefill_common.hpp).  Eight wavefronts of two column tiles per
// workgroup, one workgroup per CU, the tiles loaded straight from memory
// into LDS four steps ahead, a barrier every four steps.
//
// Measured on MI355X, chunked prefill at 8K context (bench events, A/B on
// one box at each change): one wavefront per query tile without LDS
// sharing 1,105 us; four wavefronts per workgroup, a barrier every step
// 804 us, every two steps 750 us; eight wavefronts per workgroup at one
// workgroup per CU 647 -> 615 us; eight LDS step buffers, a barrier every
// four steps 620 -> 604 us; the tiles loaded straight into LDS instead of
// staged through registers 598 -> 588 us; the QK operand's rows permuted so
// that the scores need no lane exchange 600 -> 586 us, and their K slots
// permuted against bank conflicts 589 -> 583 us.  Not kept: four column
// tiles per wavefront with the accumulators in AGPRs (1,416 us), one column
// tile per wavefront at three workgroups per CU (1,008 against 802 us),
// wave priority raised around the matrix-core instructions, the second
// half of the wavefronts delayed or run a phase behind (ping-pong), the
// operands read from LDS where they are used, and the next step's QK issued
// among a step's exponentials.
#include "prefill_common.hpp"

namespace pa {
namespace {

using namespace prefill;

// ---------------------------------------------------------------------------
// Long query runs (chunked prefill): one workgroup of W wavefronts per query
// block of W query tiles, sharing each step's K and V through LDS
// ---------------------------------------------------------------------------
// With one wavefront per query tile every tile streams the whole context
// through its own registers: each 16 KiB bf16 step feeds only 32 MFMA
// columns, and the L2 delivers the same tiles once per query tile.  Here
// the W wavefronts of a workgroup take consecutive query tiles of one
// (sequence, KV head); each step's tiles are read from memory once, by all
// lanes of the workgroup (one 16-byte piece of K and one of V each), with
// loads that write LDS directly (global_load_lds_dwordx4: lane l of a
// wavefront writes the l-th 16 bytes from the wavefront's LDS address), and
// every wavefront builds its MFMA operands from LDS in the register layout
// of the multi-query step (prefill_common.hpp's QK, softmax and PV, with
// the QK operand's rows permuted).  Eight step buffers: at the start of
// every four steps each lane issues the loads of the four steps after
// them, into the buffers the four steps before were read from; before the
// barrier that ends the four steps it waits for them.

// One LDS step buffer: K as [token group m][chunk][16 tokens] of 16-byte
// pieces, the tokens of group 1 permuted (position ^ 4) so that the tokens
// t and t + 16 one permuted operand read takes fall in distinct banks; V
// as [dimension][4 pieces of 8 tokens] with the pieces of a row permuted
// (XOR with bits 2-3 of the dimension) so that the 16 rows one lane group
// reads fall in distinct banks.
template <int D>
struct LdsStep {
  u32x4 k[2][D / 8][16];
  u32x4 v[D][4];
};

typedef __attribute__((address_space(3))) void* lds_void;

template <int CK, int D, int BS, int NT, int W>
__global__ __launch_bounds__(64 * W) void prefill_lds(const PrefillArgs args) {
  static_assert(CK == kBF16, "the LDS-shared prefill takes bf16 caches");
  using C = Cfg<CK, D, BS>;
  constexpr int kThreads = 64 * W;
  constexpr int kPieces = 2 * (D / 8) * 16;  // 16-byte pieces of K (and of V) per step
  static_assert(kPieces % 64 == 0 && kPieces <= kThreads, "one piece of K and one of V per lane and step");
  const DecodeArgs& a = args.d;
  const Item it = locate_item(a, args.tiles);
  if (!it.ok) return;  // the whole workgroup: uniform
  const int b = it.b, h = it.h, part = it.part;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int rows_w = 16 * NT / a.group;  // query rows of one wavefront
  const TileRange tr = tile_range(args, b, it.sub, part, rows_w * W);
  if (tr.i0 >= tr.nq) return;
  if (a.partition > 0 && tr.t0 >= tr.need) return;
  const int t0 = tr.t0, t1 = tr.t1;

  // this wavefront's rows of the block (none for a wavefront past its end)
  const int wi0 = tr.i0 + wave * rows_w;
  const int wi1 = min(wi0 + rows_w, tr.i1);
  const bool mine = wi0 < wi1;
  const float c2 = a.scale * kLog2e;
  Columns<CK, D, BS, NT> cols;
  if (mine) cols.init(a, tr.r0, wi0, wi1, tr.first_pos, h, col, grp, c2);
  // last token any of this wavefront's rows sees
  const int wlast = mine ? min(tr.first_pos + wi1 - 1, t1 - 1) : -1;

  // eight buffers as separate variables: the compiler then waits for a
  // buffer's own loads only
  __shared__ LdsStep<D> l0, l1, l2, l3, l4, l5, l6, l7;
  if (t0 < t1) {
    const char* kc = reinterpret_cast<const char*>(a.k_cache);
    const char* vc = reinterpret_cast<const char*>(a.v_cache);
    // block-table entries through the constant address space: scalar loads
    typedef const __attribute__((address_space(4))) int32_t* const_i32;
    const const_i32 table = (const_i32)a.block_tables + (size_t)b * a.max_blocks;
    const int nsteps = (t1 - t0 + kStep - 1) / kStep;
    const int lb_last = (t1 - 1) / BS;
    auto tile_of = [&](int lb) -> int64_t {
      int p = table[lb];
      p = (p < 0 || (int64_t)p >= a.num_blocks) ? 0 : p;
      return ((int64_t)p * a.num_kv_heads + h) * C::kTile;
    };
    struct Tiles { int64_t t0, t1; };
    auto locate = [&](int step) -> Tiles {
      const int lb0 = (t0 + step * kStep) / BS;
      const int64_t tile0 = tile_of(lb0);
      return {tile0, C::kBlocksPerStep == 2 ? tile_of(min(lb0 + 1, lb_last)) : tile0};
    };
    // This lane's pieces, as slot tid of each tensor's buffer: K slot (m,
    // chunk, position) holds token position ^ 4 m of token group m; V slot
    // (dimension, position) holds the 8-token group position ^ bits 2-3 of
    // the dimension.
    const bool carries = tid < kPieces;  // whole wavefronts
    const int km = tid / (kPieces / 2), kchunk = (tid / 16) % (D / 8), ktok = (tid % 16) ^ (km << 2);
    const int vdim = tid >> 2, vg8 = (tid & 3) ^ ((vdim >> 2) & 3);
    const int64_t koff0 = BS == 16 ? (kchunk * 16 + ktok) * 16 : (kchunk * 32 + 16 * km + ktok) * 16;
    const int64_t voff0 = BS == 16 ? vdim * 32 + (vg8 & 1) * 16 : vdim * 64 + vg8 * 16;
    const bool k_second = BS == 16 && km;
    const bool v_second = BS == 16 && (vg8 >> 1);
    // a step's K and V pieces, straight from memory into buffer L (each
    // wavefront writes 64 consecutive slots)
    auto dma = [&](const Tiles& tl, LdsStep<D>& L) {
      if (carries) {
        const int64_t kt = k_second ? tl.t1 : tl.t0;
        const int64_t vt = v_second ? tl.t1 : tl.t0;
        __builtin_amdgcn_global_load_lds(kc + kt + koff0, (lds_void)(&L.k[0][0][0] + wave * 64), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vc + vt + voff0, (lds_void)(&L.v[0][0] + wave * 64), 16, 0, 0);
      }
    };
    const int vsw = grp ^ (col >> 2);  // this lane's V piece position in its rows
    // QK A-operand rows of this lane, permuted (the step's kPermRows):
    // tokens 8 (col / 4) + col % 4 and that + 4, as (token group, K slot
    // position): the 16 lanes of a row then read 16 distinct bank groups
    int kgm[2], kpos[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int t = 8 * (col >> 2) + 4 * m + (col & 3);
      kgm[m] = t >> 4;
      kpos[m] = (t & 15) ^ (kgm[m] << 2);
    }
    StepBuf<CK, D, BS> sb;
    auto compute = [&](const LdsStep<D>& L, int step) {
      const int base = t0 + step * kStep;
      if (mine && base <= wlast) {  // a step no row of this wavefront reaches is skipped
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int j = 0; j < C::kKLoads; ++j) sb.k[m][j] = L.k[kgm[m]][grp + 4 * j][kpos[m]];
#pragma unroll
        for (int dt = 0; dt < C::kDTiles; ++dt) sb.v[dt].w = L.v[16 * dt + col][vsw];
        cols.template step<true>(sb, base, t1, grp, c2);
      }
    };
    // step n in buffer n % 8; the loads of four steps in flight while the
    // four before them are computed; a barrier every four steps
    auto load4 = [&](int s, LdsStep<D>& w0, LdsStep<D>& w1, LdsStep<D>& w2, LdsStep<D>& w3) {
      if (s < nsteps) dma(locate(s), w0);
      if (s + 1 < nsteps) dma(locate(s + 1), w1);
      if (s + 2 < nsteps) dma(locate(s + 2), w2);
      if (s + 3 < nsteps) dma(locate(s + 3), w3);
    };
    load4(0, l0, l1, l2, l3);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    auto four_steps = [&](int step, LdsStep<D>& c0, LdsStep<D>& c1, LdsStep<D>& c2_, LdsStep<D>& c3,
                          LdsStep<D>& w0, LdsStep<D>& w1, LdsStep<D>& w2, LdsStep<D>& w3) {
      load4(step + 4, w0, w1, w2, w3);
      compute(c0, step);
      if (step + 1 < nsteps) compute(c1, step + 1);
      if (step + 2 < nsteps) compute(c2_, step + 2);
      if (step + 3 < nsteps) compute(c3, step + 3);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    };
    for (int step = 0; step < nsteps; step += 8) {
      four_steps(step, l0, l1, l2, l3, l4, l5, l6, l7);
      if (step + 4 >= nsteps) break;
      four_steps(step + 4, l4, l5, l6, l7, l0, l1, l2, l3);
    }
  }
  if (mine) cols.finish(a, part, grp, c2, 1.0f);
}

// Query rows per workgroup of the LDS-shared prefill, and whether a launch
// takes it: bf16 cache with query runs long enough to fill a workgroup.
// Eight wavefronts of two column tiles per workgroup, one workgroup per CU
// (226 VGPRs: two wavefronts per SIMD; 128 KiB of LDS).
constexpr int kLdsWaves = 8;
constexpr int kLdsNT = 2;

template <int D, int BS>
hipError_t launch_lds(const PrefillArgs& p, hipStream_t stream) {
  const DecodeArgs& a = p.d;
  const int rows = 16 * kLdsNT * kLdsWaves / a.group;
  const int tiles = (p.max_query_len + rows - 1) / rows;
  const int parts = a.partition ? a.max_parts : 1;
  const long long pairs = (long long)a.num_seqs * a.num_kv_heads;
  const long long groups = (pairs + kXcds - 1) / kXcds * kXcds * parts * tiles;
  if (groups > INT32_MAX) return hipErrorInvalidValue;
  PrefillArgs q = p;
  q.tiles = tiles;
  hipLaunchKernelGGL((prefill_lds<kBF16, D, BS, kLdsNT, kLdsWaves>), dim3((unsigned)groups),
                     dim3(64 * kLdsWaves), 0, stream, q);
  return hipGetLastError();
}

}  // namespace

bool prefill_uses_lds(Elem cache, int group, int max_query_len) {
  return cache == Elem::BF16 &&
         (long long)group * max_query_len >= 16 * kLdsNT * kLdsWaves;
}

hipError_t launch_prefill_lds(const PrefillArgs& p, int head_dim, int block_size, hipStream_t stream) {
  if (head_dim == 128 && block_size == 16) return launch_lds<128, 16>(p, stream);
  if (head_dim == 128 && block_size == 32) return launch_lds<128, 32>(p, stream);
  if (head_dim == 64 && block_size == 16) return launch_lds<64, 16>(p, stream);
  if (head_dim == 64 && block_size == 32) return launch_lds<64, 32>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
