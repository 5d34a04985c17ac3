// GGUF file reader (host only).
//
// Layout from "llama.cpp AI LLM Engine - how it works" ("GGUF format"
// reference: magic "GGUF", format version, tensor count, key count; key /
// value pairs as name, value type, value, arrays led by element type and
// count; per tensor its name, up to four dimensions, element type and offset
// from the start of the data block that follows the metadata; only the
// current version, 3, is read) and from the loading page's stages (header
// parsed without tensor data, a name -> location map with duplicates
// rejected, data mapped or read on demand, split files merged into one
// map).  The numeric codes and the alignment rule, which the pages leave
// out, are those of the public GGUF specification (listed in ubd.h).
#pragma once

#include <cstdint>
#include <map>
#include <string>
#include <vector>

namespace ubd {

enum GgufValueType : int32_t {
    GV_U8 = 0, GV_I8 = 1, GV_U16 = 2, GV_I16 = 3, GV_U32 = 4, GV_I32 = 5, GV_F32 = 6,
    GV_BOOL = 7, GV_STR = 8, GV_ARR = 9, GV_U64 = 10, GV_I64 = 11, GV_F64 = 12,
};
enum GgufTensorType : int32_t { GT_F32 = 0, GT_F16 = 1, GT_Q8_0 = 8, GT_BF16 = 30 };

struct GgufValue {
    int32_t type = -1;
    int32_t etype = -1;               // arrays: element type
    uint64_t n = 0;                   // arrays: element count
    // scalars and array elements, by kind (nested arrays keep only n)
    std::vector<int64_t> i;           // integer and bool types
    std::vector<double> f;            // f32 / f64
    std::vector<std::string> s;       // strings
};

struct GgufTensor {
    std::string name;
    int32_t n_dims = 0;
    int64_t ne[4] = {1, 1, 1, 1};
    int32_t type = -1;
    uint64_t offset = 0;              // from the start of the data block
    uint64_t nbytes = 0;
};

class GgufFile {
public:
    GgufFile() = default;
    GgufFile(const GgufFile &) = delete;
    GgufFile &operator=(const GgufFile &) = delete;
    ~GgufFile();
    // Parses header, metadata and tensor records.  False (with *err) for a
    // file that is not valid GGUF version 3.
    bool open(const std::string &path, std::string *err);
    // Maps the whole file read-only (for zero-copy tensor reads).
    const uint8_t *map(std::string *err);
    // Reads a tensor's bytes into dst (nbytes of them).
    bool read(const GgufTensor &t, void *dst, std::string *err) const;

    std::string path;
    uint32_t version = 0;
    uint64_t file_size = 0, alignment = 32, data_start = 0;
    std::vector<std::string> keys;
    std::vector<GgufValue> values;
    std::map<std::string, int64_t> key_index;
    std::vector<GgufTensor> tensors;
    std::map<std::string, int64_t> tensor_index;

    const GgufValue *find(const std::string &key) const;
    bool get_int(const std::string &key, int64_t *out) const;
    bool get_float(const std::string &key, double *out) const;
    bool get_str(const std::string &key, std::string *out) const;

private:
    int fd_ = -1;
    uint8_t *map_ = nullptr;
};

// Bytes per block and values per block of a tensor type; false if unknown.
bool gguf_type_size(int32_t type, uint64_t *block_bytes, uint64_t *block_values);
const char *gguf_type_name(int32_t type);

}  // namespace ubd
