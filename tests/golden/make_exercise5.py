"""Write exercise5_online_softmax.json from closed forms (no library call).

Source of the problem: "4.4 Writing GPU Kernels with Triton", section
"Exercises", exercise 5 -- one query row, two key blocks of one key each,
already-scaled scores S1 = 2 and S2 = 4, values v1 = 1 and v2 = 3 (head
dimension 1), state starting at m = -inf, l = 0, O = 0. The page poses the
exercise without printing the answer; the numbers below are its exact
solution, written as closed forms:

  after block 1: m = 2, l = 1, O = v1 = 1
  block 2: m' = 4, alpha = e^(2-4) = e^-2
           l  = alpha * 1 + e^(4-4) = 1 + e^-2
           O  = alpha * 1 + 1 * 3   = 3 + e^-2     (un-normalised)
  O / l = (1 + 3 e^2) / (1 + e^2) = 3 - 2 / (1 + e^2)
  LSE   = ln(e^2 + e^4)          = 4 + ln(1 + e^-2)
  softmax weights (1 / (1 + e^2), 1 / (1 + e^-2))
"""
import json
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def main():
    e = math.e
    data = {
        "citation": "4.4 Writing GPU Kernels with Triton, section Exercises, exercise 5 "
                    "(worked online-softmax example; answer derived in closed form)",
        "scores": [2.0, 4.0],
        "values": [1.0, 3.0],
        "after_block1": {"m": 2.0, "l": 1.0, "O": 1.0},
        "after_block2": {"m": 4.0, "alpha": math.exp(-2.0), "l": 1.0 + math.exp(-2.0),
                         "O": 3.0 + math.exp(-2.0)},
        "O_normalised": 3.0 - 2.0 / (1.0 + e * e),
        "lse": 4.0 + math.log1p(math.exp(-2.0)),
        "weights": [1.0 / (1.0 + e * e), 1.0 / (1.0 + math.exp(-2.0))],
    }
    with open(os.path.join(HERE, "exercise5_online_softmax.json"), "w") as f:
        json.dump(data, f, indent=2)
        f.write("\n")


if __name__ == "__main__":
    main()
