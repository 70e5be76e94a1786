// Host-side evaluation of rocRAND's Philox4x32-10 engine (from its public header),
// used only to pin the oracle's Philox to an independent implementation.
// Reads N records of (ctr[4], key[2]) uint32 from argv[1], writes N x 4 uint32 to argv[2].
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
#include <cstdint>
#include <vector>

struct Probe : rocrand_device::philox4x32_10_engine {
    uint4 run(uint4 c, uint2 k) { return ten_rounds(c, k); }
};

int main(int argc, char** argv) {
    if (argc != 3) return 2;
    FILE* f = std::fopen(argv[1], "rb");
    if (!f) return 3;
    std::vector<uint32_t> in;
    uint32_t buf[6];
    while (std::fread(buf, 4, 6, f) == 6) in.insert(in.end(), buf, buf + 6);
    std::fclose(f);
    size_t n = in.size() / 6;
    std::vector<uint32_t> out(4 * n);
    Probe p;
    for (size_t i = 0; i < n; ++i) {
        uint4 c = {in[6 * i + 0], in[6 * i + 1], in[6 * i + 2], in[6 * i + 3]};
        uint2 k = {in[6 * i + 4], in[6 * i + 5]};
        uint4 r = p.run(c, k);
        out[4 * i + 0] = r.x; out[4 * i + 1] = r.y; out[4 * i + 2] = r.z; out[4 * i + 3] = r.w;
    }
    FILE* g = std::fopen(argv[2], "wb");
    if (!g) return 4;
    std::fwrite(out.data(), 4, out.size(), g);
    std::fclose(g);
    return 0;
}
