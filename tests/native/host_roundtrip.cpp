// Host-side round trip of the packed image under AddressSanitizer and UBSan:
// the library's encoder, packer and unpacker (no GPU code) on CSR and fixed-slot
// side records, N = 2 to 8, an empty matrix and a truncated image.  Exit status
// 0 when every case round-trips and the truncated image is rejected.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "stagq.h"

// A finite normal fp16 bit pattern of magnitude between about 2^-10 and 2^-4
// (the weights' scale), random sign.
static uint16_t rand_half(std::mt19937& rng) {
  const uint32_t sign = rng() & 1u, expo = 5u + rng() % 7u, mant = rng() & 0x3ffu;
  return uint16_t((sign << 15) | (expo << 10) | mant);
}

static int run(int R, int C, int g, int N, double frac, int ppr, int slots, unsigned seed) {
  std::mt19937 rng(seed);
  const int64_t n = int64_t(R) * C;
  std::vector<uint16_t> w(size_t(n) + 1);
  for (int64_t i = 0; i < n; i++) w[size_t(i)] = rand_half(rng);
  const int64_t K = int64_t(frac * double(n) + 0.5);
  const int64_t cap = K + int64_t(R) * ppr + 1;
  std::vector<uint8_t> q(size_t(n) + 1), planes(size_t(N - 2) * size_t(n) + 1);
  std::vector<uint16_t> lo(size_t(n / g) + 1), s(size_t(n / g) + 1), val(static_cast<size_t>(cap));
  std::vector<int32_t> rp(size_t(R) + 1), col(static_cast<size_t>(cap));
  int64_t npre = 0;
  int st = stagq_encode(w.data(), R, C, g, N, K, 4.0, ppr, q.data(), planes.data(), lo.data(), s.data(),
                        rp.data(), col.data(), val.data(), &npre);
  if (st) { printf("encode: status %d\n", st); return 1; }
  const int64_t nnz = rp[size_t(R)];
  stagq_fields f{R, C, g, N, q.data(), planes.data(), lo.data(), s.data(), rp.data(), col.data(), val.data(),
                 nnz, nullptr, slots};
  const size_t bytes = stagq_packed_bytes(&f);
  if (!bytes) { printf("packed_bytes: 0\n"); return 1; }
  void* img = aligned_alloc(16, (bytes + 15) / 16 * 16);
  st = stagq_pack_host(&f, img, bytes);
  if (st) { printf("pack_host: status %d\n", st); free(img); return 1; }
  stagq_info info;
  std::vector<uint8_t> q2(q.size()), p2(planes.size());
  std::vector<uint16_t> lo2(lo.size()), s2(s.size()), v2(val.size());
  std::vector<int32_t> rp2(rp.size()), c2(col.size());
  st = stagq_unpack_host(img, bytes, &info, q2.data(), p2.data(), lo2.data(), s2.data(), rp2.data(), c2.data(),
                         v2.data());
  if (st) { printf("unpack_host: status %d\n", st); free(img); return 1; }
  bool ok = memcmp(q.data(), q2.data(), size_t(n)) == 0 &&
            memcmp(planes.data(), p2.data(), size_t(N - 2) * size_t(n)) == 0 &&
            memcmp(lo.data(), lo2.data(), size_t(n / g) * 2) == 0 && memcmp(s.data(), s2.data(), size_t(n / g) * 2) == 0 &&
            rp == rp2 && memcmp(col.data(), c2.data(), size_t(nnz) * 4) == 0 &&
            memcmp(val.data(), v2.data(), size_t(nnz) * 2) == 0;
  if (stagq_unpack_host(img, bytes - 1, &info, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == 0) {
    printf("a truncated image was accepted\n");
    ok = false;
  }
  printf("%d x %d g=%d N=%d nnz=%lld side_slots=%d: %s\n", R, C, g, N, (long long)nnz, info.side_slots,
         ok ? "round trip ok" : "MISMATCH");
  free(img);
  return ok ? 0 : 1;
}

int main() {
  int bad = 0;
  bad |= run(37, 384, 64, 4, 0.01, 0, 0, 1);
  bad |= run(37, 384, 64, 4, 0.01, 0, -1, 2);
  bad |= run(40, 512, 32, 6, 0.02, 3, -1, 3);
  bad |= run(16, 256, 128, 2, 0.0, 0, -1, 4);
  bad |= run(33, 1024, 128, 8, 0.005, 2, 7, 6);
  bad |= run(0, 256, 128, 4, 0.0, 0, 0, 7);
  return bad;
}
