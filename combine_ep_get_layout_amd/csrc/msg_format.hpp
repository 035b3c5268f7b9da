// Message body format shared by the packer (messages.hip) and the receiver
// (receive.hip): a 16-byte header {s, d, n, body bytes}, the body
// codes | scales | weights | expert ids | source token (each section
// zero-padded to 16 bytes), then a 16-byte completion flag {epoch, 0, 0, 0}.
// Descriptor fields are big-endian.
#pragma once

#include "ep_internal.hpp"

namespace ep {

struct MsgSections {
  int64_t off[5];  // section offsets within the body
  int64_t len[5];  // unpadded section lengths
  int64_t body;    // body bytes (sum of padded sections)
};

__host__ __device__ inline int64_t pad16(int64_t v) { return (v + 15) & ~(int64_t)15; }

// Body of a message with n tokens: codes | scales | weights | ids | token.
__host__ __device__ inline MsgSections msg_sections(int64_t n, int H, int K, int quant) {
  MsgSections m;
  const int64_t G = H / 128;
  m.len[0] = n * H * (quant == EP_QUANT_NONE ? 2 : 1);
  m.len[1] = n * G * (quant == EP_QUANT_FP8_F32 ? 4 : (quant == EP_QUANT_FP8_UE8M0 ? 1 : 0));
  m.len[2] = n * K * 4;
  m.len[3] = n * K * 4;
  m.len[4] = n * 4;
  int64_t o = 0;
  for (int i = 0; i < 5; ++i) {
    m.off[i] = o;
    o += pad16(m.len[i]);
  }
  m.body = o;
  return m;
}

__device__ __forceinline__ uint32_t be32(uint32_t v) { return __builtin_bswap32(v); }

// Keys: rank << 16 | region index.  Region indices above kMaxRegionIndex do
// not fit; such a piece gets kBadKey (rank 0xFFFF, never a valid rank).
constexpr int64_t kMaxRegionIndex = 0xFFFF;
constexpr uint32_t kBadKey = 0xFFFFFFFFu;

}  // namespace ep
