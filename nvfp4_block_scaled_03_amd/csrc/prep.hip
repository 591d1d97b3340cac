// Offline weight rearrangement into the grouped GEMMs' streaming layout.
//
// For an expert matrix W [N][K] (canonical NVFP4: codes [N][K/2], scales
// [N][K/16]) the layout is, per expert:
//   codes : [N/16 column tiles][K/128 chunks][64 lanes][16 bytes]
//   scales: [N/32 tile pairs][K/128/G chunk groups][64 lanes][G chunks][2 tiles][2 bytes]
// Lane l = 16*g + n of a (tile, chunk) holds the 32 codes k in
// [32g, 32g + 32) of the chunk for column n of the tile, in canonical nibble
// order, and the two scale bytes of those k; the scale bytes of the two
// tiles of a pair sit side by side, and those of G consecutive chunks
// (G = 4, 3, 2 or 1, the largest dividing K/128) follow each other, so a lane
// fetches the scales of a tile pair for G chunks with one load of 4G bytes.
// One wavefront therefore reads a
// whole (tile, chunk) with one coalesced 16-byte load per lane, and every
// lane's bytes are exactly the operand fragment it feeds to the 16x16x32
// matrix instruction (8 codes per k-step).  All experts' codes come first,
// then all experts' scales.
//
// Gate/up weights (interleave_I = I > 0): column tile 2q holds gate rows
// [16q, 16q + 16) and tile 2q + 1 the up rows [I + 16q, I + 16q + 16), so a
// wavefront that owns a tile pair holds matching gate and up columns and can
// apply SwiGLU in registers.
#include "common.h"
#include "launch.h"

namespace nvfp4 {
namespace {

__global__ __launch_bounds__(256) void prep_kernel(int64_t slots, int64_t N, int64_t K,
                                                   int64_t interleave_I,
                                                   const uint8_t* __restrict__ q,
                                                   const uint8_t* __restrict__ sf,
                                                   uint8_t* __restrict__ prep) {
  const int64_t KC = K / 128, NT = N / 16;
  const int64_t pieces = slots * NT * KC * 64;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= pieces) return;
  const int64_t lane = i & 63;
  int64_t rest = i >> 6;
  const int64_t kc = rest % KC;
  rest /= KC;
  const int64_t nt = rest % NT;
  const int64_t e = rest / NT;
  const int64_t n = lane & 15, g = lane >> 4;
  int64_t row;
  if (interleave_I > 0) {
    const int64_t qt = nt >> 1;
    row = (nt & 1) ? interleave_I + 16 * qt + n : 16 * qt + n;
  } else {
    row = nt * 16 + n;
  }
  const uint8_t* src = q + (e * N + row) * (K / 2) + kc * 64 + 16 * g;
  const u32x4 v = *reinterpret_cast<const u32x4*>(src);
  *reinterpret_cast<u32x4*>(prep + i * 16) = v;
  const uint8_t* ssrc = sf + (e * N + row) * (K / 16) + kc * 8 + 2 * g;
  uint8_t* sdst = prep + slots * N * (K / 2) + e * (N / 32) * KC * 256 +
                  scale_word_offset(nt >> 1, (int)kc, (int)KC, (int)lane) + (nt & 1) * 2;
  sdst[0] = ssrc[0];
  sdst[1] = ssrc[1];
}

}  // namespace

size_t prep_bytes(int64_t slots, int64_t N, int64_t K) {
  return (size_t)(slots * N * (K / 2) + slots * N * (K / 16));
}

hipError_t launch_prep(int64_t slots, int64_t N, int64_t K, int interleave_I, const uint8_t* q,
                       const uint8_t* sf, uint8_t* prep, hipStream_t s) {
  const int64_t pieces = slots * (N / 16) * (K / 128) * 64;
  const int64_t blocks = (pieces + 255) / 256;
  prep_kernel<<<(unsigned)blocks, 256, 0, s>>>(slots, N, K, interleave_I, q, sf, prep);
  return hipGetLastError();
}

}  // namespace nvfp4
