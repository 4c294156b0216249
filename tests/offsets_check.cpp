// Host-side check of the buffer offsets that the compact small-message
// two-stage kernel takes instead of pointers (tensor_all_reduce_amd/csrc/
// ar_offsets.hpp).  Built with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_offsets.py; addresses are
// made up and never dereferenced.  Prints "offsets check: ok" when every
// case holds.
#include <cstdint>
#include <cstdio>

#include "ar_offsets.hpp"

static int fails = 0;
#define CHECK(c)                                                  \
  do {                                                            \
    if (!(c)) {                                                   \
      std::printf("FAIL line %d: %s\n", __LINE__, #c);            \
      ++fails;                                                    \
    }                                                             \
  } while (0)

static const uintptr_t kBase = 0x100000000000ull;  // 16 TiB: room for +-2 TiB without wrapping

// Packs base + rel[i] (rel[0] = 0); when it fits, checks that every rebuilt
// address is the original and that unused slots are zero.  Returns whether
// it fit; *shift receives the unit's exponent.
static bool pack(const int64_t* rel, int count, unsigned* shift) {
  const void* p[2 * AR_MAX_RANKS];
  for (int i = 0; i < count; ++i) p[i] = reinterpret_cast<const void*>(kBase + static_cast<uintptr_t>(rel[i]));
  ar::PtrOffsets po;
  if (!ar::pack_offsets(p, count, &po)) return false;
  CHECK(po.base == static_cast<const char*>(p[0]));
  for (int i = 1; i < count; ++i) CHECK(ar::offset_address(po, i - 1) == static_cast<const char*>(p[i]));
  for (int i = count - 1; i < 2 * AR_MAX_RANKS - 1; ++i) CHECK(po.off[i] == 0);
  *shift = po.shift;
  return true;
}

int main() {
  const int64_t G = 1ll << 30;
  unsigned s = 99;

  // sixteen separately allocated 256 MiB buffers, 2 MiB apart beyond that
  {
    int64_t rel[16];
    for (int i = 0; i < 16; ++i) rel[i] = i * (256ll << 20) + i * (2ll << 20);
    CHECK(pack(rel, 16, &s) && s == 21);
  }
  // the unit is the largest power of two dividing every difference
  {
    const int64_t rel[] = {0, 48, 16, -32};
    CHECK(pack(rel, 4, &s) && s == 4);
    const int64_t rel2[] = {0, 3 * 512, -7 * 1024};
    CHECK(pack(rel2, 3, &s) && s == 9);
  }
  // reach in 16-byte units: INT32_MAX and INT32_MIN units fit, one more does not
  {
    const int64_t hi[] = {0, 16, INT32_MAX * 16ll};
    CHECK(pack(hi, 3, &s) && s == 4);
    const int64_t hi1[] = {0, 16, (INT32_MAX + 1ll) * 16};
    CHECK(!pack(hi1, 3, &s));
    const int64_t lo[] = {0, 16, INT32_MIN * 16ll};
    CHECK(pack(lo, 3, &s) && s == 4);
    const int64_t lo1[] = {0, 16, (INT32_MIN - 1ll) * 16};
    CHECK(!pack(lo1, 3, &s));
  }
  // alone, a far buffer with many trailing zero bits fits through a large unit
  {
    const int64_t far[] = {0, 1ll << 35};
    CHECK(pack(far, 2, &s) && s == 30);
    const int64_t far_neg[] = {0, -(1ll << 35), 3 * G};
    CHECK(pack(far_neg, 3, &s) && s == 30);
  }
  // the unit stops at 2^30: differences that are multiples of 2^32 use 2^30
  {
    const int64_t rel[] = {0, 4 * G, 12 * G, -8 * G};
    CHECK(pack(rel, 4, &s) && s == 30);
  }
  // 2 TiB away at 2^30 units is 2^11 units: fits; 2^31 units does not
  {
    const int64_t ok[] = {0, 2048 * G};
    CHECK(pack(ok, 2, &s) && s == 30);
    const int64_t no[] = {0, 16, (1ll << 31) * 16};
    CHECK(!pack(no, 3, &s));
  }
  // an output equal to an input (partial aliasing) is a repeated offset
  {
    const int64_t rel[] = {0, 1 << 20, 2 << 20, 1 << 20};
    CHECK(pack(rel, 4, &s) && s == 20);
  }
  // P = 1: one input and one output
  {
    const int64_t rel[] = {0, -4096};
    CHECK(pack(rel, 2, &s) && s == 12);
  }
  // every count from 1 to 2 * AR_MAX_RANKS; outside that range nothing packs
  for (int count = 1; count <= 2 * AR_MAX_RANKS; ++count) {
    int64_t rel[2 * AR_MAX_RANKS];
    for (int i = 0; i < count; ++i) rel[i] = (i % 2 ? -1 : 1) * i * (1ll << 24) + i * 16;
    CHECK(pack(rel, count, &s));
  }
  {
    const void* p[1] = {reinterpret_cast<const void*>(kBase)};
    ar::PtrOffsets po;
    CHECK(!ar::pack_offsets(p, 0, &po));
    const void* q[2 * AR_MAX_RANKS + 1] = {};
    CHECK(!ar::pack_offsets(q, 2 * AR_MAX_RANKS + 1, &po));
  }
  // the struct is 72 bytes, so with n the argument segment is 80
  CHECK(sizeof(ar::PtrOffsets) == 72);

  if (fails == 0) std::printf("offsets check: ok\n");
  return fails == 0 ? 0 : 1;
}
