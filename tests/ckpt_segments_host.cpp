// Host build of the segment-boundary and sequence-range helpers (kda_ckpt.h)
// for tests/test_ckpt_segments.py.
#include "kda_ckpt.h"

extern "C" int kda_test_segments(const int32_t* offs, int C, int len, int* lo_hi, int cap) {
  const kda::CkptList k{offs, 0, C, len};
  const int nseg = (len + 63) / 64 + kda::count_cuts(k);
  if (nseg > cap) return -1;
  for (int j = 0; j < nseg; ++j) {
    lo_hi[2 * j] = j == 0 ? 0 : kda::interior_boundary(k, j - 1);
    lo_hi[2 * j + 1] = j == nseg - 1 ? len : kda::interior_boundary(k, j);
  }
  return nseg;
}

extern "C" int kda_test_walk(const int32_t* offs, int C, int len, int* ends, int cap) {
  const kda::CkptList k{offs, 0, C, len};
  int n = 0;
  for (int p = 0; p < len; p = kda::next_boundary(k, p)) {
    if (n >= cap) return -1;
    ends[n++] = kda::next_boundary(k, p);
  }
  return n;
}

extern "C" int kda_test_honoured(const int32_t* offs, int C, int len, int* mask) {
  const kda::CkptList k{offs, 0, C, len};
  for (int c = 0; c < C; ++c) mask[c] = 0;
  int n = 0;
  kda::for_each_honoured(k, [&](int c, int) {
    mask[c] = 1;
    ++n;
  });
  return n;
}

extern "C" void kda_test_seq_range(int64_t b, int64_t e, int64_t T_total, int64_t* bos_len) {
  kda::clamp_seq_range(b, e, T_total, &bos_len[0], &bos_len[1]);
}
